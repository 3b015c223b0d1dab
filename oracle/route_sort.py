"""CPU oracle for the MoE route-sort path.  TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The product path (the HIP library and its Python binding) never
calls it, and this module shares no code with that path.

What the path computes comes from the page "Kimi-K3 B1 route-sort +
prepared-MoE handoff (stack)", Summary section: router logits are converted to
FP32, a per-expert correction bias is added, a grouped top-k picks the experts,
and "both sort phases" turn the picks into expert-sorted metadata that the
grouped GEMM reads directly.  The metadata format (per-expert histogram,
exclusive prefix sum of block-padded counts, scatter of token-slot ids t*k+j
with sentinel M*k, expert id per block, total padded rows) is the one the
route-sort contract of this library defines.  The page "gfx1250 ordinary-TP
route optimization" (Capacity and dispatch; Dispatch and contracts; Tests and
compatibility) supplies the route-row invariants used by the checkers below:
exact counts, a row-slot bijection and per-expert ownership.

Readings taken where the pages are silent:
  * scoring is the logistic sigmoid, s = RN32(1 / (1 + exp(-x))), correctly
    rounded to FP32;
  * the correction bias is added to the score used for choosing,
    key = RN32(s + b); the routing weights use the unbiased s;
  * groups are contiguous blocks of E / n_group experts; a group's score is the
    FP32 sum of its two largest keys (the single key when a group has one
    expert);
  * groups are ranked by (score desc, group index asc), experts by (key desc,
    expert index asc);
  * out_ids[t] lists the k chosen experts in ascending expert id;
  * weights are s / sum(s) over the k picks, evaluated in float64;
  * within an expert's segment the token-slot ids are ascending (stable).

Parity status: every function here is pinned by tests/test_oracle_pins.py,
tests/test_oracle_gap_pins.py (the near-tie gaps) and
tests/test_oracle_counter_pins.py (initial counters): exhaustive, brute-force,
closed-form, hand-worked or invariant checks.  Whether the
readings above match the pages' own kernel cannot be checked from the pages,
which print no worked example.
"""
from __future__ import annotations

import dataclasses
import decimal
from typing import List, Optional

import numpy as np

F32 = np.float32
F64 = np.float64


# ---------------------------------------------------------------------------
# Step a1: FP32 conversion of the logits ("FP32-logit conversion", Summary).
# ---------------------------------------------------------------------------
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """BF16 is the top half of an FP32 word: widening is a 16-bit left shift."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def logits_to_f32(storage: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f32(storage)
    if dtype == "f32":
        return np.asarray(storage, dtype=np.float32)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Step a2: sigmoid score, correctly rounded to FP32.
# ---------------------------------------------------------------------------
_DEC_CTX = decimal.Context(prec=60)


def _sigmoid_decimal(x: float) -> decimal.Decimal:
    d = decimal.Decimal(float(x))  # exact value of the float
    return _DEC_CTX.divide(decimal.Decimal(1), _DEC_CTX.add(decimal.Decimal(1), _DEC_CTX.exp(-d)))


def _round_decimal_to_f32(v: decimal.Decimal, guess: np.float32) -> np.float32:
    """Nearest FP32 to the decimal value v, searching the neighbours of guess."""
    cands = [np.nextafter(np.nextafter(guess, F32(-np.inf)), F32(-np.inf)),
             np.nextafter(guess, F32(-np.inf)), guess,
             np.nextafter(guess, F32(np.inf)),
             np.nextafter(np.nextafter(guess, F32(np.inf)), F32(np.inf))]
    best, best_err = None, None
    for c in cands:
        if not np.isfinite(c) or c < 0:
            continue
        err = abs(decimal.Decimal(float(c)) - v)
        if best_err is None or err < best_err or (
                err == best_err and (int(np.float32(c).view(np.uint32)) & 1) == 0):
            best, best_err = np.float32(c), err
    return best


def sigmoid_f32(x: np.ndarray) -> np.ndarray:
    """s = RN32(1 / (1 + exp(-x))) for FP32 x, correctly rounded.

    The logistic function is evaluated in float64 (relative error a few units
    of 2^-53).  Where that result lies so close to the midpoint between two
    FP32 neighbours that the float64 error could flip the rounding, the value
    is recomputed with 60-digit decimal arithmetic and rounded exactly.
    """
    x = np.asarray(x, dtype=np.float32)
    x64 = x.astype(np.float64)
    with np.errstate(over="ignore"):
        r = 1.0 / (1.0 + np.exp(-x64))
    s = r.astype(np.float32)
    # distance of r to the two FP32 rounding boundaries around s
    up = np.nextafter(s, F32(np.inf)).astype(np.float64)
    dn = np.nextafter(s, F32(-np.inf)).astype(np.float64)
    s64 = s.astype(np.float64)
    mid_up = 0.5 * (s64 + up)
    mid_dn = 0.5 * (s64 + dn)
    tol = np.abs(r) * 2.0 ** -45 + 2.0 ** -1000
    risky = (np.abs(r - mid_up) <= tol) | (np.abs(r - mid_dn) <= tol)
    if np.any(risky):
        flat_x = x.reshape(-1)
        flat_s = s.reshape(-1)
        for i in np.flatnonzero(risky.reshape(-1)):
            flat_s[i] = _round_decimal_to_f32(_sigmoid_decimal(float(flat_x[i])), flat_s[i])
        s = flat_s.reshape(x.shape)
    return s


def biased_keys(x_f32: np.ndarray, bias: np.ndarray):
    """key = RN32(s + b): the correction bias is added to the score used for
    choosing ("correction bias", Summary); returns (s, key)."""
    s = sigmoid_f32(x_f32)
    key = (s + np.asarray(bias, dtype=np.float32)).astype(np.float32)
    return s, key


# ---------------------------------------------------------------------------
# Steps a3-a5: grouped top-k ("grouped top-k", Summary).
# ---------------------------------------------------------------------------
def group_scores(key_row: np.ndarray, n_group: int) -> np.ndarray:
    """Score of each contiguous group: FP32 sum of its two largest keys."""
    E = key_row.shape[0]
    G = E // n_group
    kg = key_row.reshape(n_group, G)
    if G == 1:
        return kg[:, 0].astype(np.float32)
    top = -np.sort(-kg, axis=1)  # descending per group
    return (top[:, 0] + top[:, 1]).astype(np.float32)


def rank_desc(values: np.ndarray) -> np.ndarray:
    """Indices ordered by (value desc, index asc)."""
    idx = np.arange(values.shape[0])
    return np.lexsort((idx, -values.astype(np.float64)))


@dataclasses.dataclass
class TokenRoute:
    ids: np.ndarray          # [k] int32 ascending
    groups: np.ndarray       # selected group indices, ascending
    gap_k: Optional[float]   # key_(k) - key_(k+1) among allowed experts
    gap_g: Optional[float]   # gs_(topk_group) - gs_(topk_group+1)


def route_token(key_row: np.ndarray, n_group: int, topk_group: int, k: int) -> TokenRoute:
    E = key_row.shape[0]
    G = E // n_group
    gs = group_scores(key_row, n_group)
    gorder = rank_desc(gs)
    kept = np.sort(gorder[:topk_group])
    gap_g = None
    if topk_group < n_group:
        gap_g = float(gs[gorder[topk_group - 1]]) - float(gs[gorder[topk_group]])
    allowed = np.concatenate([np.arange(g * G, (g + 1) * G) for g in kept])
    order = allowed[rank_desc(key_row[allowed])]
    chosen = order[:k]
    gap_k = None
    if allowed.shape[0] > k:
        gap_k = float(key_row[order[k - 1]]) - float(key_row[order[k]])
    return TokenRoute(np.sort(chosen).astype(np.int32), kept.astype(np.int32), gap_k, gap_g)


def route_weights(s_row: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """w_j = s_{id_j} / sum of s over the k picks, evaluated in float64."""
    sv = s_row[ids].astype(np.float64)
    return sv / sv.sum()


# ---------------------------------------------------------------------------
# Steps a6-a8: "both sort phases" -> dispatch metadata.
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class SortMeta:
    counts: np.ndarray           # [E] routes per expert (the histogram)
    padded: np.ndarray           # [E] counts rounded up to a multiple of block
    offsets: np.ndarray          # [E] exclusive prefix sum of padded
    num_post_pad: int
    sorted_ids: np.ndarray       # [num_post_pad] token-slot ids, sentinel M*k
    expert_of_block: np.ndarray  # [num_post_pad // block]


def sort_metadata(ids: np.ndarray, E: int, block: int) -> SortMeta:
    """Counting sort of token slots s = t*k + j by expert, stable in s.

    A slot whose id lies outside [0, E) is a dropped route: it claims no row
    and its slot number appears nowhere in sorted_ids (page "gfx1250
    ordinary-TP route optimization", Dispatch and contracts: negative expert
    ids claim no slot; ids past E are not counted).  The sentinel stays M*k."""
    ids = np.asarray(ids, dtype=np.int64)
    M, k = ids.shape
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E).astype(np.int64)   # phase 1
    padded = (counts + block - 1) // block * block
    offsets = np.concatenate([[0], np.cumsum(padded)[:-1]]).astype(np.int64)
    num_post_pad = int(padded.sum())
    slots = np.flatnonzero(valid)                                      # phase 2
    order = slots[np.argsort(flat[valid], kind="stable")]
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64)
    sorted_ids = np.full(num_post_pad, M * k, dtype=np.int64)
    for e in range(E):
        c = counts[e]
        if c:
            sorted_ids[offsets[e]:offsets[e] + c] = order[starts[e]:starts[e] + c]
    expert_of_block = np.repeat(np.arange(E, dtype=np.int64), padded // block)
    return SortMeta(counts, padded, offsets, num_post_pad,
                    sorted_ids.astype(np.int32), expert_of_block.astype(np.int32))


@dataclasses.dataclass
class CounterMeta:
    meta: SortMeta               # counts / padded / offsets include the initial counters
    written: np.ndarray          # [num_post_pad] bool: rows this call writes
    counters_out: np.ndarray     # [E] initial + this call's routes


def sort_metadata_counters(ids: np.ndarray, E: int, block: int, initial: np.ndarray) -> CounterMeta:
    """The sort phases with caller-provided per-expert counters (page "gfx1250
    ordinary-TP route optimization", Dispatch and contracts: counters that
    the caller hands in start from the values it gave them).

    initial[e] >= 0 counts rows the caller already holds at the head of expert
    e's segment.  The segment then covers initial[e] + (this call's routes to
    e) rows, padded to a multiple of block; offsets are the exclusive prefix of
    the padded sizes; this call's r-th route to e (ascending slot order, ids
    outside [0, E) dropped) lands on row offsets[e] + initial[e] + r; the
    caller's rows [offsets[e], offsets[e] + initial[e]) are not written; the
    rest of the segment is the sentinel M*k.  The counters advance to initial
    + routes."""
    ids = np.asarray(ids, dtype=np.int64)
    M, k = ids.shape
    c0 = np.asarray(initial, dtype=np.int64)
    assert c0.shape == (E,) and np.all(c0 >= 0)
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    routes = np.bincount(flat[valid], minlength=E).astype(np.int64)
    counts = c0 + routes
    padded = (counts + block - 1) // block * block
    offsets = np.concatenate([[0], np.cumsum(padded)[:-1]]).astype(np.int64)
    num_post_pad = int(padded.sum())
    sorted_ids = np.full(num_post_pad, M * k, dtype=np.int64)
    written = np.ones(num_post_pad, dtype=bool)
    for e in range(E):
        written[offsets[e]:offsets[e] + c0[e]] = False
        mine = np.flatnonzero(valid & (flat == e))  # ascending slots
        sorted_ids[offsets[e] + c0[e]:offsets[e] + c0[e] + mine.size] = mine
    sorted_ids[~written] = -1
    expert_of_block = np.repeat(np.arange(E, dtype=np.int64), padded // block)
    meta = SortMeta(counts, padded, offsets, num_post_pad, sorted_ids.astype(np.int32),
                    expert_of_block.astype(np.int32))
    return CounterMeta(meta, written, counts.astype(np.int64))


def local_metadata(ids: np.ndarray, local_begin: int, local_count: int, block: int) -> SortMeta:
    """Sort metadata of one expert-parallel rank that owns experts
    [local_begin, local_begin + local_count), numbered from 0 there.  A route
    to another rank's expert claims no row here, like a dropped route (page
    "gfx1250 ordinary-TP route optimization", Dispatch and contracts); the
    sentinel stays M*k."""
    ids = np.asarray(ids, dtype=np.int64)
    rel = ids - local_begin
    rel = np.where((rel >= 0) & (rel < local_count), rel, -1)
    return sort_metadata(rel, local_count, block)


# ---------------------------------------------------------------------------
# The whole path.
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class RouteResult:
    ids: np.ndarray          # [M, k] int32
    weights: np.ndarray      # [M, k] float64
    meta: SortMeta
    s: np.ndarray            # [M, E] float32 sigmoid scores
    keys: np.ndarray         # [M, E] float32 biased keys
    gap_k: np.ndarray        # [M] float64 (inf where undefined)
    gap_g: np.ndarray        # [M] float64 (inf where undefined)


def route_sort(logits_storage: np.ndarray, dtype: str, bias: np.ndarray, k: int,
               n_group: int, topk_group: int, block: int,
               tokens: Optional[np.ndarray] = None) -> RouteResult:
    """Reference for the whole hot path.  `tokens` restricts the selection to a
    subset of rows (for sampled checks of large inputs); the sort metadata is
    then built from those rows only."""
    x = logits_to_f32(logits_storage, dtype)
    if tokens is not None:
        x = x[np.asarray(tokens)]
    M, E = x.shape
    s, keys = biased_keys(x, bias)
    ids = np.zeros((M, k), dtype=np.int32)
    w = np.zeros((M, k), dtype=np.float64)
    gap_k = np.full(M, np.inf)
    gap_g = np.full(M, np.inf)
    for t in range(M):
        r = route_token(keys[t], n_group, topk_group, k)
        ids[t] = r.ids
        w[t] = route_weights(s[t], r.ids)
        if r.gap_k is not None:
            gap_k[t] = r.gap_k
        if r.gap_g is not None:
            gap_g[t] = r.gap_g
    meta = sort_metadata(ids, E, block)
    return RouteResult(ids, w, meta, s, keys, gap_k, gap_g)


# ---------------------------------------------------------------------------
# Invariant checkers (used on oracle output and on GPU output alike).
# ---------------------------------------------------------------------------
def check_sort_invariants(ids: np.ndarray, sorted_ids: np.ndarray, expert_of_block: np.ndarray,
                          num_post_pad: int, E: int, block: int) -> List[str]:
    """Route-row invariants: exact counts, padding with the sentinel M*k, a
    bijection of real rows onto token slots, one expert per block, ascending
    slots within an expert.  Returns the list of violated properties."""
    errs = []
    ids = np.asarray(ids, dtype=np.int64)
    M, k = ids.shape
    sentinel = M * k
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)  # ids outside [0, E) are dropped routes
    nvalid = int(valid.sum())
    counts = np.bincount(flat[valid], minlength=E) if nvalid else np.zeros(E, np.int64)
    if counts.sum() != nvalid:
        errs.append("histogram does not sum to the number of routed slots")
    if num_post_pad % block != 0:
        errs.append("num_post_pad not a multiple of block")
    if num_post_pad != int(((counts + block - 1) // block * block).sum()):
        errs.append("num_post_pad differs from sum of padded counts")
    rows = np.asarray(sorted_ids[:num_post_pad], dtype=np.int64)
    eob = np.asarray(expert_of_block[: num_post_pad // block], dtype=np.int64)
    if rows.shape[0] != num_post_pad or eob.shape[0] != num_post_pad // block:
        errs.append("metadata shorter than num_post_pad")
        return errs
    real = rows[rows != sentinel]
    if real.shape[0] != nvalid or not np.array_equal(np.sort(real), np.flatnonzero(valid)):
        errs.append("real rows are not a bijection onto the routed token slots")
        return errs
    if np.any((rows < 0) | (rows > sentinel)):
        errs.append("row value out of range")
    if eob.size and (np.any(eob < 0) or np.any(eob >= E)):
        errs.append("expert_of_block out of range")
    if eob.size > 1 and np.any(np.diff(eob) < 0):
        errs.append("expert_of_block not non-decreasing")
    nblk = np.bincount(eob, minlength=E) if eob.size else np.zeros(E, np.int64)
    if not np.array_equal(nblk, (counts + block - 1) // block):
        errs.append("blocks per expert differ from ceil(count/block)")
    blk_of_row = np.arange(num_post_pad) // block
    is_real = rows != sentinel
    if np.any(flat[rows[is_real]] != eob[blk_of_row[is_real]]):
        errs.append("a block holds a slot of another expert")
    # within each expert segment: real rows first and ascending, then sentinels
    seg_start = 0
    for e in range(E):
        p = int((counts[e] + block - 1) // block * block)
        seg = rows[seg_start:seg_start + p]
        c = int(counts[e])
        if np.any(seg[c:] != sentinel) or np.any(seg[:c] == sentinel):
            errs.append(f"expert {e}: sentinels not confined to the segment tail")
            break
        if c > 1 and np.any(np.diff(seg[:c]) <= 0):
            errs.append(f"expert {e}: slots not ascending")
            break
        seg_start += p
    return errs


def check_selection_invariants(keys: np.ndarray, ids: np.ndarray, n_group: int,
                               topk_group: int) -> List[str]:
    """Each token has k distinct ascending ids, all inside its topk_group best
    groups, and every chosen key beats every unchosen allowed key (ties go to
    the lower index)."""
    errs = []
    M, E = keys.shape
    k = ids.shape[1]
    G = E // n_group
    for t in range(M):
        row = ids[t].astype(np.int64)
        if np.any(np.diff(row) <= 0) or row.min() < 0 or row.max() >= E:
            errs.append(f"token {t}: ids not distinct/ascending/in range")
            continue
        gs = group_scores(keys[t], n_group)
        gorder = rank_desc(gs)
        kept = set(int(g) for g in gorder[:topk_group])
        if any(int(e) // G not in kept for e in row):
            errs.append(f"token {t}: id outside the best groups")
            continue
        allowed = np.array([e for e in range(E) if e // G in kept])
        chosen = set(int(e) for e in row)
        worst = min(row, key=lambda e: (float(keys[t, e]), -int(e)))
        for e in allowed:
            if int(e) in chosen:
                continue
            if (float(keys[t, e]), -int(e)) > (float(keys[t, worst]), -int(worst)):
                errs.append(f"token {t}: unchosen expert {e} beats chosen {worst}")
                break
    return errs
