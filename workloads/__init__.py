"""Seeded synthetic inputs for the MoE route-sort path.

This module only draws random numbers and packs them into the storage formats
the path accepts (FP32, or BF16 bit patterns).  It holds none of the method's
arithmetic: no sigmoid, no bias add, no selection and no sorting.  Both the CPU
oracle's tests and the GPU path's tests/benchmark take their inputs from here.

The workload shapes follow the pages' Kimi-K3 TP8 routing (896 routed experts,
top-16; "Kimi-K3 B1 route-sort + prepared-MoE handoff (stack)", Summary, and
"gfx1250 ordinary-TP route optimization", Capacity and dispatch section).  The
pages measure on real model routing, which is not available here; these seeded
distributions stand in for it.

Draw order for every workload: logits (standard normal, [M, E]), then the
per-expert offsets (if the recipe has them), then the correction bias.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class RouteConfig:
    name: str
    M: int            # tokens
    E: int            # routed experts
    k: int            # experts per token
    n_group: int      # expert groups (contiguous blocks of E // n_group experts)
    topk_group: int   # groups kept per token
    block: int        # padding granularity of each expert's segment
    dtype: str        # storage type of the logits: "f32" or "bf16"
    dist: str         # logit distribution recipe (see make_logits)
    bias_range: float  # bias ~ U(-bias_range, bias_range)
    seed: int = 0

    @property
    def routes(self) -> int:
        return self.M * self.k


# The five workloads: a tiny case, batch-1 decode, the histogram-threshold
# batch, a skewed prefill chunk and the widest expert set (4096 experts, the
# 16 KiB LDS histogram limit).
CONFIGS: Dict[str, RouteConfig] = {
    "tiny": RouteConfig("tiny", 4, 64, 4, 8, 4, 16, F32, "normal", 0.1),
    "decode": RouteConfig("decode", 1, 896, 16, 8, 4, 32, BF16, "normal", 0.1),
    "threshold": RouteConfig("threshold", 512, 896, 16, 1, 1, 64, BF16, "offset_normal", 0.1),
    "prefill_skew": RouteConfig("prefill_skew", 8192, 896, 16, 8, 4, 128, BF16, "log_zipf", 0.1),
    "wide": RouteConfig("wide", 16384, 4096, 16, 16, 8, 128, F32, "normal", 0.2),
}
CONFIG_ORDER = ["tiny", "decode", "threshold", "prefill_skew", "wide"]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round FP32 values to BF16 (round to nearest, ties to even); return the
    16-bit patterns as uint16.  Storage packing of generated inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def make_logits(rng: np.random.Generator, M: int, E: int, dist: str) -> np.ndarray:
    """FP32 logits [M, E] for one of the recipes below."""
    base = rng.standard_normal((M, E), dtype=np.float32)
    if dist == "normal":
        return base
    if dist == "offset_normal":
        # uneven expert load: a per-expert offset ~ N(0, 0.5) drawn once
        off = rng.normal(0.0, 0.5, size=E).astype(np.float32)
        return base + off[None, :]
    if dist == "log_zipf":
        # expert popularity rank r (1 = hottest) from a seeded permutation;
        # offset = -1.1 * ln(r): Zipf(s=1.1) weights in log space
        r = rng.permutation(E).astype(np.float64) + 1.0
        off = (-1.1 * np.log(r)).astype(np.float32)
        return base + off[None, :]
    if dist == "hot":
        # one hot expert (+8) on top of N(0,1)
        hot = int(rng.integers(0, E))
        base[:, hot] += np.float32(8.0)
        return base
    if dist == "shared":
        # "shared" expert: one expert with a large offset, the rest random
        hot = int(rng.integers(0, E))
        base[:, hot] += np.float32(4.0)
        return base
    if dist == "dominant_group":
        # the first eighth of the experts is shifted up by 1.5
        base[:, : max(1, E // 8)] += np.float32(1.5)
        return base
    if dist == "equal":
        # every logit identical: all keys tie except for the bias
        return np.zeros((M, E), dtype=np.float32)
    if dist == "duplicated":
        # experts come in pairs with identical logits (bias is duplicated too,
        # see make_bias), so exact key ties must be broken by index
        half = base[:, : (E + 1) // 2]
        return np.repeat(half, 2, axis=1)[:, :E].copy()
    if dist == "coarse":
        # logits on a coarse grid (multiples of 1/4 in [-4, 4]): many exact ties
        return np.clip(np.round(base * 4.0) / 4.0, -4.0, 4.0).astype(np.float32)
    raise ValueError(f"unknown logit distribution {dist!r}")


def make_bias(rng: np.random.Generator, E: int, bias_range: float, dist: str = "normal") -> np.ndarray:
    b = rng.uniform(-bias_range, bias_range, size=E).astype(np.float32)
    if dist == "duplicated":
        b = np.repeat(b[: (E + 1) // 2], 2)[:E].copy()
    if dist == "equal":
        b = np.zeros(E, dtype=np.float32)
    return b


@dataclasses.dataclass
class RouteInputs:
    cfg: RouteConfig
    logits_f32: np.ndarray            # [M, E] FP32 values the path sees (BF16 already applied)
    logits_storage: np.ndarray        # [M, E] float32 or uint16 (BF16 bit patterns)
    bias: np.ndarray                  # [E] float32


def make_inputs(cfg: RouteConfig, seed: Optional[int] = None) -> RouteInputs:
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    x = make_logits(rng, cfg.M, cfg.E, cfg.dist)
    b = make_bias(rng, cfg.E, cfg.bias_range, cfg.dist)
    if cfg.dtype == BF16:
        bits = f32_to_bf16_bits(x)
        vals = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
        return RouteInputs(cfg, vals, bits, b)
    if cfg.dtype == F32:
        return RouteInputs(cfg, x, x, b)
    raise ValueError(cfg.dtype)


def custom(M: int, E: int, k: int, n_group: int, topk_group: int, block: int,
           dtype: str = F32, dist: str = "normal", bias_range: float = 0.1,
           seed: int = 0, name: str = "custom") -> RouteConfig:
    return RouteConfig(name, M, E, k, n_group, topk_group, block, dtype, dist, bias_range, seed)


def logits_bytes(cfg: RouteConfig) -> int:
    return cfg.M * cfg.E * (2 if cfg.dtype == BF16 else 4)
