"""Seeded synthetic inputs for the Multi-Token Attention forward layer.

This module is shared by the tests, the benchmark and the oracle harness. It only
draws random numbers and converts storage formats; it performs none of the
layer's arithmetic (no logits, convolution, softmax, mixing or normalisation).

Workload recipe (every array is produced by ``numpy.random.default_rng(seed)``):

* draw order: q, k, v (each ``[B, T, M, d]``, standard normal, float32), then the
  key-query kernel noise ``[M, c_q, c_k]``, then the head-mixing noise
  ``[M/c_h, c_h, c_h]``, then (long-context workload only) the planted key pairs;
  a placement on both sides of softmax draws a leading axis of 2 (before, after);
* ``theta = delta(0, centre) + sigma_theta * noise``; ``w = I + sigma_w * noise``
  (sigma is a standard deviation), on each side;
* bf16 workloads round q, k, v to bfloat16 (round-to-nearest-even) once, after
  planting; both the GPU and the oracle then see the identical rounded values.

Shapes follow the 880M-model layer described on the page "Multi-Token Attention |
Summary" (Appendix D: hidden size 1536, 16 heads, context 2048) and its kernel
sizes (§4.2: c_q=6, c_k=11); no dataset item is used.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "MTAConfig",
    "CONFIGS",
    "config",
    "make_inputs",
    "round_bf16",
    "bf16_bits",
    "bits_to_float",
    "sample_rows",
]


@dataclasses.dataclass(frozen=True)
class MTAConfig:
    """One synthetic workload. ``kq``/``mix`` are ``"pre"``, ``"post"``, ``"both"`` or ``None``."""

    name: str
    B: int
    T: int
    M: int
    d: int
    c_q: int
    c_k: int
    c_h: int
    kq: Optional[str]
    mix: Optional[str]
    gn: bool
    dtype: str  # "bf16" or "fp32"
    theta_sigma: float
    w_sigma: float
    gamma: float = 1.0
    beta: float = 0.0
    lam: float = 1.0
    seed: int = 0
    plant_block: int = 0  # >0: one correlated key pair per block of this many tokens
    plant_gap: int = 5
    plant_rho: float = 0.9

    def replace(self, **kw) -> "MTAConfig":
        return dataclasses.replace(self, **kw)

    @property
    def tokens(self) -> int:
        return self.B * self.T


# The five workloads. Unstated details (seed of configs 1-4, the noise of configs 3-4,
# the GroupNorm values of configs 1 and 3, the kernel sizes of config 2, the planting
# correlation) are this library's readings of the workload descriptions.
CONFIGS = [
    MTAConfig("tiny_fp32", 1, 64, 4, 16, 3, 5, 2, "pre", "post", True, "fp32",
              0.1, 0.1, 1.0, 0.0, 0.8, seed=0),
    MTAConfig("slice880m_bf16", 4, 2048, 16, 96, 6, 11, 2, "pre", "post", True, "bf16",
              0.05, 0.05, 1.0, 0.0, 0.8, seed=1),
    MTAConfig("degenerate_bf16", 4, 2048, 16, 128, 6, 11, 2, "pre", "post", False, "bf16",
              0.0, 0.0, seed=2),
    MTAConfig("longctx_bf16", 1, 16384, 16, 128, 6, 11, 4, "pre", "post", True, "bf16",
              0.05, 0.05, 1.0, 0.0, 0.8, seed=3, plant_block=512),
    MTAConfig("variant_bf16", 2, 4096, 32, 128, 4, 9, 4, "post", "pre", True, "bf16",
              0.05, 0.05, 1.0, 0.0, 1.0 / math.sqrt(12.0), seed=4),
    # Both convolutions on both sides of softmax (the experiments' default placement, §4
    # of the page) at the T=4096 shape above.
    MTAConfig("both_sides_bf16", 2, 4096, 32, 128, 4, 9, 4, "both", "both", True, "bf16",
              0.05, 0.05, 1.0, 0.0, 1.0 / math.sqrt(12.0), seed=5),
]


def config(idx_or_name) -> MTAConfig:
    if isinstance(idx_or_name, int):
        return CONFIGS[idx_or_name]
    for c in CONFIGS:
        if c.name == idx_or_name:
            return c
    raise KeyError(idx_or_name)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bits = bits + 0x7FFF + ((bits >> 16) & 1)
    out = (bits & 0xFFFF0000).astype(np.uint32)
    return out.view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def bits_to_float(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_inputs(cfg: MTAConfig) -> dict:
    """Draw the seeded inputs of ``cfg``. Returns float32 arrays (bf16-exact for bf16)."""
    rng = np.random.default_rng(cfg.seed)
    shape = (cfg.B, cfg.T, cfg.M, cfg.d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    sides_kq = (2,) if cfg.kq == "both" else ()
    sides_mix = (2,) if cfg.mix == "both" else ()
    theta_noise = rng.standard_normal(sides_kq + (cfg.M, cfg.c_q, cfg.c_k), dtype=np.float32)
    w_noise = rng.standard_normal(sides_mix + (cfg.M // cfg.c_h, cfg.c_h, cfg.c_h), dtype=np.float32)

    if cfg.plant_block > 0:
        blk, gap, rho = cfg.plant_block, cfg.plant_gap, cfg.plant_rho
        n_blocks = cfg.T // blk
        for b in range(cfg.B):
            for n in range(n_blocks):
                p = int(rng.integers(n * blk, n * blk + blk - gap))
                z = rng.standard_normal((cfg.M, cfg.d), dtype=np.float32)
                k[b, p + gap] = np.float32(rho) * k[b, p] + np.float32(math.sqrt(1.0 - rho * rho)) * z

    theta = (cfg.theta_sigma * theta_noise).astype(np.float32)
    theta[..., 0, (cfg.c_k - 1) // 2] += np.float32(1.0)
    w = (cfg.w_sigma * w_noise).astype(np.float32)
    for u in range(cfg.c_h):
        w[..., u, u] += np.float32(1.0)

    if cfg.dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    gamma = np.full(cfg.M * cfg.d, cfg.gamma, dtype=np.float32)
    beta = np.full(cfg.M * cfg.d, cfg.beta, dtype=np.float32)
    return dict(q=q, k=k, v=v, theta=theta, w=w, gamma=gamma, beta=beta,
                lam=float(np.float32(cfg.lam)))


def sample_rows(T: int, row_tile: int = 0, n_random: int = 24, seed: int = 12345) -> np.ndarray:
    """Query rows to check at sizes the oracle cannot finish in full.

    Covers the first and last rows, rows around multiples of ``row_tile`` (tile
    edges and their halo) and a few seeded random rows.
    """
    rows = set(range(min(T, 12)))
    rows.update(range(max(0, T - 12), T))
    if row_tile > 0:
        for t in range(row_tile, T, row_tile * max(1, (T // row_tile) // 6)):
            for dr in (-3, -1, 0, 1, 2):
                if 0 <= t + dr < T:
                    rows.add(t + dr)
    rng = np.random.default_rng(seed)
    rows.update(int(x) for x in rng.integers(0, T, size=n_random))
    return np.array(sorted(rows), dtype=np.int32)
