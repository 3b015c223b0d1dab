"""CPU oracle for the grouped GEMM that consumes the route-sort metadata.
TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The product path never calls it, and this module shares no code
with that path.

The page "Kimi-K3 B1 route-sort + prepared-MoE handoff (stack)", Summary,
says the route-sort output is prepared for the first grouped GEMM and read by
it directly, with no second top-k or sort.  This is that first GEMM written
out from its definition over the metadata:

  for every sorted row r < num_post_pad, with slot s = sorted_ids[r] and
  expert e = expert_of_block[r // block]:
      y[r, :] = x[s // k, :] . W[e]^T      when s < M*k (a real route),
      y[r, :] = 0                          when s is the sentinel M*k.

Shapes follow the page "gfx1250 ordinary-TP route optimization", Capacity and
dispatch (the tested Kimi-K3 TP8 MoE: 896 experts, top-16, routed hidden size
K = 3584, intermediate size I = 384 per rank, BF16 output).

Readings taken where the pages are silent:
  * the first GEMM computes the gate and up projections together, so W[e] is
    [N, K] with N = 2*I (the page's activation takes a gate and an up input);
  * x and W are BF16, products are accumulated exactly here (float64 of BF16
    values: every product is exact and the K-term sums are far inside float64
    precision), the kernel accumulates in FP32 and rounds the result to BF16
    (round to nearest even);
  * padding rows are written as zeros, rows at or beyond num_post_pad are
    not written.

Parity status: pinned by tests/test_oracle_gemm_pins.py (integer-valued
inputs against an integer dense product, closed forms with selection and
constant matrices, sentinel rows, sampled rows against the full result).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """BF16 patterns (uint16) to float64; BF16 is the top half of an FP32 word."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _row_sources(sorted_ids: np.ndarray, expert_of_block: np.ndarray, rows: np.ndarray,
                 M: int, k: int, block: int):
    """Token and expert of each listed sorted row; token -1 for a padding row."""
    s = np.asarray(sorted_ids, dtype=np.int64)[rows]
    e = np.asarray(expert_of_block, dtype=np.int64)[rows // block]
    tok = np.where((s >= 0) & (s < M * k), s // k, -1)
    return tok, e


def gemm1_rows(x_bits: np.ndarray, w_bits: np.ndarray, sorted_ids: np.ndarray,
               expert_of_block: np.ndarray, M: int, k: int, block: int,
               rows: Sequence[int]) -> np.ndarray:
    """y for the listed sorted rows only, float64 [len(rows), N].

    x_bits: [M, K] uint16 (BF16), w_bits: [E, N, K] uint16 (BF16)."""
    rows = np.asarray(rows, dtype=np.int64)
    E, N, K = w_bits.shape
    tok, e = _row_sources(sorted_ids, expert_of_block, rows, M, k, block)
    out = np.zeros((rows.size, N), dtype=np.float64)
    # one matrix product per expert over that expert's listed rows
    for ex in np.unique(e[tok >= 0]):
        sel = np.nonzero((e == ex) & (tok >= 0))[0]
        xa = bf16_to_f64(x_bits[tok[sel]])           # [n, K]
        wa = bf16_to_f64(w_bits[ex])                 # [N, K]
        out[sel] = xa @ wa.T
    return out


def gemm1_sorted(x_bits: np.ndarray, w_bits: np.ndarray, sorted_ids: np.ndarray,
                 expert_of_block: np.ndarray, num_post_pad: int, M: int, k: int,
                 block: int) -> np.ndarray:
    """y for every sorted row below num_post_pad, float64 [num_post_pad, N]."""
    return gemm1_rows(x_bits, w_bits, sorted_ids, expert_of_block, M, k, block,
                      np.arange(int(num_post_pad)))


def abs_products(x_bits: np.ndarray, w_bits: np.ndarray, sorted_ids: np.ndarray,
                 expert_of_block: np.ndarray, M: int, k: int, block: int,
                 rows: Sequence[int]) -> np.ndarray:
    """sum_i |x_i| |w_i| for every listed output element: the scale of the
    rounding error of any summation order of the same products."""
    return gemm1_rows(np.asarray(x_bits) & np.uint16(0x7FFF), np.asarray(w_bits) & np.uint16(0x7FFF),
                      sorted_ids, expert_of_block, M, k, block, rows)


def f64_to_bf16_bits(y: np.ndarray) -> np.ndarray:
    """Round float64 values to BF16 (through FP32, each step to nearest even)."""
    u = np.asarray(y, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def tolerance(ref: np.ndarray, absprod: np.ndarray, K: int) -> np.ndarray:
    """Largest allowed |y_kernel - y_exact| for a BF16 result of an FP32
    accumulation of K exact products: the FP32 sum of K terms in any order is
    within (K - 1) * 2^-24 * sum|x_i w_i| of the exact sum (each addition
    rounds once, relative error 2^-24, on a partial sum bounded by
    sum|x_i w_i|), and rounding that to BF16 moves it by at most half a BF16
    unit of the FP32 value, 2^-8 of its magnitude."""
    acc = (K - 1) * 2.0 ** -24 * absprod
    return acc + 2.0 ** -8 * (np.abs(ref) + acc)
