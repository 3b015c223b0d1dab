"""CPU oracle for the router gate projection in front of the route-sort path.
TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The product path never calls it, and this module shares no code
with that path.

The page "Kimi-K3 B1 route-sort + prepared-MoE handoff (stack)", Summary,
lists a specialised batch-1 gate projection directly in front of the
route-sort kernel, which starts from FP32 router logits.  The gate is the
linear map logits[t, e] = sum_i hidden[t, i] * W[e, i].

Readings taken where the pages are silent:
  * hidden states and gate weights are BF16 ([M, H] and [E, H], row-major);
    the hidden size H is a parameter (the pages give the model hidden size
    7168 for Kimi-K3);
  * the FP32 logit is the exact dot product rounded once to FP32 (round to
    nearest, ties to even).  Every BF16 x BF16 product is exact in float64,
    math.fsum returns the correctly rounded float64 sum, and the one case
    where rounding that to FP32 could differ from rounding the exact sum (the
    float64 sum sitting exactly on an FP32 rounding midpoint) is settled with
    exact rational arithmetic.

Parity status: pinned by tests/test_oracle_gate_pins.py (integer inputs,
selection weights, a constructed midpoint case, agreement with a float64
matrix product within its error bound).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _round_to_f32(s64: float, exact_terms: np.ndarray) -> np.float32:
    """RN32 of the exact sum whose correctly rounded float64 value is s64."""
    r = np.float32(s64)
    if not math.isfinite(s64):
        return r
    # neighbours of r in FP32 and the midpoints next to it
    lo = np.nextafter(r, np.float32(-np.inf))
    hi = np.nextafter(r, np.float32(np.inf))
    for nb in (lo, hi):
        mid = (float(r) + float(nb)) / 2.0  # exact in float64
        if s64 == mid:
            exact = sum((Fraction(float(v)) for v in exact_terms), Fraction(0))
            m = Fraction(mid)
            if exact == m:
                return r  # a true tie: numpy already rounded it to even
            # the exact sum lies strictly on one side of the midpoint
            return nb if (exact > m) == (float(nb) > float(r)) else r
    return r


def gate_logits(hidden_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """FP32 logits [M, E]: each one the exact dot product rounded to FP32."""
    h = bf16_to_f64(hidden_bits)   # [M, H]
    w = bf16_to_f64(w_bits)        # [E, H]
    M, E = h.shape[0], w.shape[0]
    out = np.empty((M, E), dtype=np.float32)
    for t in range(M):
        prods = w * h[t]           # exact: 8-bit x 8-bit significands
        for e in range(E):
            out[t, e] = _round_to_f32(math.fsum(prods[e]), prods[e])
    return out


def midpoint_margin(hidden_bits: np.ndarray, w_bits: np.ndarray, logits: np.ndarray) -> np.ndarray:
    """Distance of each exact dot product from the nearest FP32 rounding
    midpoint, relative to sum |h_i w_i| (float64 estimate).  A kernel that
    accumulates in float64 can round differently from the exact value only
    where this is below its accumulation error bound."""
    h = bf16_to_f64(hidden_bits)
    w = bf16_to_f64(w_bits)
    absd = np.abs(h) @ np.abs(w).T                       # [M, E]
    exact = np.array([[math.fsum(w[e] * h[t]) for e in range(w.shape[0])] for t in range(h.shape[0])])
    r = logits.astype(np.float32)
    up = np.nextafter(r, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(r, np.float32(-np.inf)).astype(np.float64)
    rf = r.astype(np.float64)
    d = np.minimum(np.abs(exact - (rf + up) / 2), np.abs(exact - (rf + dn) / 2))
    return d / np.maximum(absd, np.finfo(np.float64).tiny)
