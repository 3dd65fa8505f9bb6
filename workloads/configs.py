"""The five synthetic DiT attention workloads.

Shapes are [B, H, L, d] with d contiguous.  Each workload names a static
block mask by generator kind and parameters; the generators themselves are
implemented twice, independently: in the C library (for the product) and in
the oracle (for checking).  Nothing here computes a mask.

Workload sources (shapes only; no model weights or prompts are used):
  1  tiny fp32 sanity case, 32x32 block grid, diagonal blocks kept.
  2  PixArt-Sigma-like 1024x1024 image: 64x64 latent tokens, 16 heads, d=72.
  3  CogVideoX-2B-like video: 226 text tokens + 13 frames of 30x45 latents,
     30 heads, d=64; 3D spatio-temporal window plus the text-block column.
  4  Hunyuan-DiT-like image: 4096 image tokens + 77 text tokens, d=88.
  5  Long-video density sweep at L=115200, H=24, d=128 (the shape of the
     per-step kernel-latency figure of the growing-sparsity paper page).
"""
from dataclasses import dataclass, field
from typing import List, Tuple

MASK_DIAG = 0
MASK_BAND = 1
MASK_COGVIDEO3D = 2
MASK_FULL = 3
MASK_CUSTOM = 99  # a mask given explicitly (tests), never built by a generator


@dataclass(frozen=True)
class MaskSpec:
    kind: int
    nb: int
    w: int = 0
    text_blocks: int = 0
    tshift: int = 0

    def label(self) -> str:
        names = {MASK_DIAG: "diag", MASK_BAND: "band", MASK_COGVIDEO3D: "cogvideo3d", MASK_FULL: "full"}
        s = f"{names.get(self.kind, 'custom')}(nb={self.nb}"
        if self.kind == MASK_BAND:
            s += f",w={self.w}"
        if self.kind == MASK_COGVIDEO3D:
            s += f",text={self.text_blocks},tshift={self.tshift}"
        return s + ")"


@dataclass(frozen=True)
class Config:
    number: int
    name: str
    B: int
    H: int
    L: int
    d: int
    block: int
    dtype: str            # "f32" or "bf16": the I/O and MFMA operand type
    masks: Tuple[MaskSpec, ...]
    sparse_steps: int     # sparse steps after each calibration
    input_scale: float = 1.0   # Q, K, V ~ N(0, input_scale^2)
    drift_sigma: float = 0.05  # absolute step of the random walk: X + N(0, drift_sigma^2) per step
    lam: float = 0.04

    @property
    def nb(self) -> int:
        return -(-self.L // self.block)

    @property
    def seed(self) -> int:
        return self.number


def _cfgs() -> dict:
    c = {}
    c[1] = Config(1, "tiny_fp32", 1, 2, 1024, 64, 32, "f32",
                  (MaskSpec(MASK_DIAG, 32),), 1, input_scale=1.0 / 8.0)
    c[2] = Config(2, "pixart_sigma_like", 2, 16, 4096, 72, 64, "bf16",
                  (MaskSpec(MASK_BAND, 64, w=2),), 4)
    c[3] = Config(3, "cogvideox2b_like", 2, 30, 17776, 64, 64, "bf16",
                  (MaskSpec(MASK_COGVIDEO3D, 278, text_blocks=4, tshift=21),), 4)
    c[4] = Config(4, "hunyuan_dit_like", 2, 16, 4173, 88, 64, "bf16",
                  (MaskSpec(MASK_BAND, 66, w=2), MaskSpec(MASK_BAND, 66, w=4)), 4)
    # window widths: round-half-up of 900 * {1/4, 1/8, 1/16, 1/32}
    c[5] = Config(5, "long_video_sweep", 1, 24, 115200, 128, 128, "bf16",
                  tuple(MaskSpec(MASK_BAND, 900, w=w) for w in (225, 113, 56, 28)), 4)
    return c


CONFIGS = _cfgs()

# Density sweep on the shapes of workload 3: band windows of round-half-up(278 * {1/4, 1/8, 1/16,
# 1/32}) key blocks per query block, i.e. 75 / 87.5 / 93.8 / 96.9% nominal block sparsity.
SWEEP_C3 = tuple(MaskSpec(MASK_BAND, 278, w=w) for w in (70, 35, 17, 9))
