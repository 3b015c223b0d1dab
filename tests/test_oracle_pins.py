"""Pins for the CPU oracle: each check ties it to something other than itself
(an exhaustive comparison with an independent routine, brute-force enumeration,
a closed form or an invariant), so that a plausible mistake anywhere in the
oracle fails at least one test.  CPU only."""
import decimal
import itertools
import math

import numpy as np
import pytest

import workloads
from oracle import route_sort as orc


# ---------------------------------------------------------------------------
# a1: BF16 -> FP32 widening, exhaustive over all 65536 patterns against torch's
# own bfloat16 conversion.
# ---------------------------------------------------------------------------
def test_bf16_widening_exhaustive_vs_torch():
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.bf16_bits_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_generator_rounding_is_nearest_even():
    # the generator's packing is storage only, but the inputs must be the BF16
    # values nearest to the FP32 draws; check against torch's conversion
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = rng.standard_normal(100000).astype(np.float32) * 10
    bits = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)


# ---------------------------------------------------------------------------
# a2: sigmoid, correctly rounded to FP32.
# ---------------------------------------------------------------------------
_CTX = decimal.Context(prec=50)


def _exact_round_sigmoid(x: float) -> np.float32:
    """Independent evaluation: 50-digit decimal sigmoid, then the nearest FP32
    found by bracketing with FP32 neighbours of a float64 estimate."""
    d = decimal.Decimal(x)
    v = _CTX.divide(1, _CTX.add(1, _CTX.exp(-d)))
    g = np.float32(float(v))
    best = None
    for c in (np.nextafter(g, np.float32(-1)), g, np.nextafter(g, np.float32(2))):
        err = abs(decimal.Decimal(float(c)) - v)
        if best is None or err < best[0]:
            best = (err, c)
    return np.float32(best[1])


def _finite_bf16_values(lo=-120.0, hi=120.0):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = orc.bf16_bits_to_f32(bits)
    x = x[np.isfinite(x)]
    return np.unique(x[(x >= lo) & (x <= hi)])


def test_sigmoid_exhaustive_bf16_vs_decimal():
    x = _finite_bf16_values()
    ours = orc.sigmoid_f32(x)
    ref = np.array([_exact_round_sigmoid(float(v)) for v in x], dtype=np.float32)
    bad = np.flatnonzero(ours.view(np.uint32) != ref.view(np.uint32))
    assert bad.size == 0, (x[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_sigmoid_fp32_sample_vs_decimal():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(3000) * 4,
                        rng.uniform(-110, 40, 1000)]).astype(np.float32)
    ours = orc.sigmoid_f32(x)
    ref = np.array([_exact_round_sigmoid(float(v)) for v in x], dtype=np.float32)
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_sigmoid_special_values_and_shape():
    s = orc.sigmoid_f32(np.array([0.0, -0.0, np.inf, -np.inf, 17.5, 40.0, -104.0, -200.0,
                                  2.0 ** -30, -(2.0 ** -30)], dtype=np.float32))
    assert s[0] == 0.5 and s[1] == 0.5
    assert s[2] == 1.0 and s[3] == 0.0
    assert s[4] == 1.0 and s[5] == 1.0          # 1 - e^-x below half an ulp of 1
    assert s[6] == 0.0 and s[7] == 0.0           # e^x below half the smallest subnormal
    assert s[8] == 0.5 and s[9] == 0.5           # 0.5 + x/4 rounds back to 0.5
    # monotone non-decreasing on a dense sorted grid
    x = np.linspace(-30, 30, 200001).astype(np.float32)
    assert np.all(np.diff(orc.sigmoid_f32(x).astype(np.float64)) >= 0)


def test_sigmoid_agrees_with_scipy_expit_on_bf16():
    """scipy's float64 expit rounded to FP32 agrees with the oracle except where
    the float64 value sits on an FP32 rounding midpoint.  That happens for tiny
    BF16 x: 0.5 + x/4 is exactly a midpoint and the cubic term (below float64
    resolution at 0.5) decides the rounding; there the decimal evaluation must
    side with the oracle."""
    special = pytest.importorskip("scipy.special")
    x = _finite_bf16_values(-200.0, 200.0)
    ours = orc.sigmoid_f32(x)
    r64 = special.expit(x.astype(np.float64))
    ref = r64.astype(np.float32)
    bad = np.flatnonzero(ours.view(np.uint32) != ref.view(np.uint32))
    for i in bad:
        lo, hi = sorted([float(ours[i]), float(ref[i])])
        assert np.nextafter(np.float32(lo), np.float32(2)) == np.float32(hi)  # one ulp apart
        assert r64[i] == 0.5 * (lo + hi)                                       # expit on the midpoint
        assert abs(float(x[i])) < 2.0 ** -15                                   # only for tiny x
        assert _exact_round_sigmoid(float(x[i])) == ours[i]
    assert bad.size < 200


def test_biased_keys_closed_form():
    # x = 0 gives s = 0.5 exactly; biases that are multiples of 2^-8 make the
    # sum exact, so key = 0.5 + b with no rounding
    b = (np.arange(-8, 9) / 256.0).astype(np.float32)
    s, key = orc.biased_keys(np.zeros(17, np.float32), b)
    assert np.all(s == 0.5)
    assert np.array_equal(key, (0.5 + b.astype(np.float64)).astype(np.float32))
    # bias added after the sigmoid, not to the logit
    s, key = orc.biased_keys(np.array([2.0], np.float32), np.array([0.5], np.float32))
    assert abs(float(key[0]) - (1 / (1 + math.exp(-2.0)) + 0.5)) < 1e-6
    # FP32 rounding of the sum: 0.5 + 2^-25 ties to even -> 0.5
    s, key = orc.biased_keys(np.zeros(1, np.float32), np.array([2.0 ** -25], np.float32))
    assert key[0] == np.float32(0.5)


# ---------------------------------------------------------------------------
# a3-a5: grouped top-k, brute force on tiny expert sets.
# ---------------------------------------------------------------------------
def _brute_force_route(key: np.ndarray, n_group: int, topk_group: int, k: int):
    """Enumerate every group subset and every expert subset and keep the
    lexicographically best by (value desc, index asc).  Group score is the best
    FP32 sum over pairs of distinct experts in the group (single key if the
    group has one expert)."""
    E = key.shape[0]
    G = E // n_group
    gs = []
    for g in range(n_group):
        mem = range(g * G, (g + 1) * G)
        if G == 1:
            gs.append(np.float32(key[g * G]))
        else:
            gs.append(max(np.float32(key[i] + key[j]) for i, j in itertools.combinations(mem, 2)))

    def best_subset(items, m, val):
        best, best_sig = None, None
        for sub in itertools.combinations(items, m):
            sig = sorted(((float(val(i)), -i) for i in sub), reverse=True)
            if best_sig is None or sig > best_sig:
                best, best_sig = sub, sig
        return sorted(best)

    groups = best_subset(range(n_group), topk_group, lambda g: gs[g])
    allowed = [e for g in groups for e in range(g * G, (g + 1) * G)]
    return best_subset(allowed, k, lambda e: key[e])


@pytest.mark.parametrize("E,n_group,topk_group,k", [
    (4, 1, 1, 2), (6, 3, 2, 2), (8, 4, 2, 3), (8, 2, 1, 4), (9, 3, 1, 2),
    (10, 5, 3, 4), (12, 4, 2, 3), (12, 6, 4, 4), (12, 12, 5, 3), (12, 3, 3, 5),
    (6, 6, 6, 6), (5, 1, 1, 5),
])
def test_grouped_topk_brute_force(E, n_group, topk_group, k):
    rng = np.random.default_rng(E * 100 + n_group * 10 + k)
    for trial in range(40):
        if trial % 4 == 0:
            # constructed exact ties: keys from a tiny value set
            key = rng.choice(np.array([0.25, 0.5, 0.75], np.float32), E)
        elif trial % 4 == 1:
            x = rng.choice(np.array([-1.0, 0.0, 1.0], np.float32), E)
            _, key = orc.biased_keys(x, np.zeros(E, np.float32))
        else:
            x = rng.standard_normal(E).astype(np.float32)
            b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
            _, key = orc.biased_keys(x, b)
        got = orc.route_token(key.astype(np.float32), n_group, topk_group, k).ids
        want = _brute_force_route(key.astype(np.float32), n_group, topk_group, k)
        assert list(got) == want, (trial, key, got, want)


def test_single_group_is_plain_stable_topk():
    rng = np.random.default_rng(5)
    for _ in range(50):
        key = rng.choice(np.linspace(0, 1, 7).astype(np.float32), 40)
        got = orc.route_token(key, 1, 1, 9).ids
        # stable sort of -key keeps equal keys in index order
        want = np.sort(np.argsort(-key.astype(np.float64), kind="stable")[:9])
        assert np.array_equal(got, want)


def test_all_groups_kept_equals_ungrouped():
    rng = np.random.default_rng(6)
    for _ in range(50):
        key = rng.standard_normal(48).astype(np.float32)
        a = orc.route_token(key, 8, 8, 7).ids
        b = orc.route_token(key, 1, 1, 7).ids
        assert np.array_equal(a, b)


def test_all_equal_keys():
    key = np.full(64, 0.625, np.float32)
    r = orc.route_token(key, 8, 4, 4)
    assert list(r.ids) == [0, 1, 2, 3]
    s = np.full(64, 0.5, np.float32)
    w = orc.route_weights(s, r.ids)
    assert np.all(w == 0.25)


def test_group_score_is_top_two_sum():
    key = np.array([0.1, 0.9, 0.5, 0.3, 0.8, 0.8, 0.0, 0.2], np.float32)
    gs = orc.group_scores(key, 2)
    assert gs[0] == np.float32(np.float32(0.9) + np.float32(0.5))
    assert gs[1] == np.float32(np.float32(0.8) + np.float32(0.8))  # duplicates count twice
    assert np.array_equal(orc.group_scores(key, 8), key)


def test_hand_worked_example():
    # E=8, two groups of four, keep one group, k=2.  Group 0 top-2 = 0.9+0.2,
    # group 1 top-2 = 0.7+0.6 -> group 1 wins although group 0 holds the
    # single best key; inside group 1 the picks are experts 5 and 6.
    key = np.array([0.9, 0.2, 0.1, 0.0, 0.5, 0.7, 0.6, 0.3], np.float32)
    r = orc.route_token(key, 2, 1, 2)
    assert list(r.groups) == [1]
    assert list(r.ids) == [5, 6]
    # group tie -> lower group index; expert tie -> lower expert index
    key = np.array([0.5, 0.5, 0.5, 0.5], np.float32)
    r = orc.route_token(key, 2, 1, 1)
    assert list(r.groups) == [0] and list(r.ids) == [0]


def test_weights_normalise_unbiased_scores():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((3, 32)).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, 32).astype(np.float32)
    res = orc.route_sort(x, "f32", b, 4, 4, 2, 8)
    for t in range(3):
        sv = res.s[t, res.ids[t]].astype(np.float64)
        assert abs(res.weights[t].sum() - 1.0) < 1e-15
        assert np.allclose(res.weights[t] * sv.sum(), sv, rtol=1e-15, atol=0)


# ---------------------------------------------------------------------------
# a6-a8: sort metadata against the definition of each output written out slot
# by slot, and the M=1 closed form.
# ---------------------------------------------------------------------------
def _metadata_by_definition(ids, E, block):
    M, k = ids.shape
    flat = [int(v) for v in ids.reshape(-1)]
    counts = [flat.count(e) for e in range(E)]
    padded = [-(-c // block) * block for c in counts]
    off = [sum(padded[:e]) for e in range(E)]
    total = sum(padded)
    rows = [M * k] * total
    for s, e in enumerate(flat):
        rank = sum(1 for s2 in range(s) if flat[s2] == e)
        rows[off[e] + rank] = s
    eob = [e for e in range(E) for _ in range(padded[e] // block)]
    return counts, total, rows, eob


@pytest.mark.parametrize("M,E,k,block", [(1, 8, 3, 4), (5, 6, 2, 1), (7, 10, 3, 3),
                                         (16, 12, 4, 5), (3, 4, 4, 8), (9, 30, 2, 16)])
def test_sort_metadata_by_definition(M, E, k, block):
    rng = np.random.default_rng(M * E + k)
    for _ in range(5):
        ids = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(M)])
        meta = orc.sort_metadata(ids, E, block)
        counts, total, rows, eob = _metadata_by_definition(ids, E, block)
        assert list(meta.counts) == counts
        assert meta.num_post_pad == total
        assert list(meta.sorted_ids) == rows
        assert list(meta.expert_of_block) == eob
        assert orc.check_sort_invariants(ids, meta.sorted_ids, meta.expert_of_block,
                                         meta.num_post_pad, E, block) == []


def test_sort_metadata_single_token_closed_form():
    ids = np.array([[3, 17, 40, 41, 100, 200, 333, 400, 401, 402, 500, 600, 700, 800, 801, 895]])
    k, block = 16, 32
    meta = orc.sort_metadata(ids, 896, block)
    assert meta.num_post_pad == k * block == 512
    assert list(meta.expert_of_block) == list(ids[0])
    want = []
    for j in range(k):
        want += [j] + [k] * (block - 1)
    assert list(meta.sorted_ids) == want


def test_sort_metadata_is_stable_counting_sort():
    rng = np.random.default_rng(9)
    ids = np.stack([np.sort(rng.choice(20, 5, replace=False)) for _ in range(300)])
    meta = orc.sort_metadata(ids, 20, 7)
    real = meta.sorted_ids[meta.sorted_ids != ids.size]
    # real rows equal the slots ordered by (expert, slot): a lexsort
    flat = ids.reshape(-1)
    assert np.array_equal(real, np.lexsort((np.arange(flat.size), flat)))


def _metadata_by_definition_dropping(ids, E, block):
    """The definition with dropped routes written out: a slot whose id is not
    in [0, E) takes no row; every other slot goes to its expert's segment in
    ascending slot order."""
    M, k = ids.shape
    flat = [int(v) for v in ids.reshape(-1)]
    keep = [0 <= e < E for e in flat]
    counts = [sum(1 for s, e in enumerate(flat) if keep[s] and e == x) for x in range(E)]
    padded = [-(-c // block) * block for c in counts]
    off = [sum(padded[:e]) for e in range(E)]
    rows = [M * k] * sum(padded)
    fill = [0] * E
    for s, e in enumerate(flat):
        if keep[s]:
            rows[off[e] + fill[e]] = s
            fill[e] += 1
    eob = [e for e in range(E) for _ in range(padded[e] // block)]
    return counts, sum(padded), rows, eob


@pytest.mark.parametrize("M,E,k,block", [(1, 8, 3, 4), (6, 6, 2, 1), (7, 10, 3, 3), (16, 12, 4, 5),
                                         (9, 30, 2, 16)])
def test_sort_metadata_drops_ids_outside_range(M, E, k, block):
    """Dropped routes (negative ids, ids >= E) claim no row and no slot; rows
    may also repeat an expert.  Checked against the definition by brute force."""
    rng = np.random.default_rng(M + 31 * E + k)
    for trial in range(6):
        ids = rng.integers(-3, E + 3, size=(M, k))
        if trial == 0:
            ids[:] = -1                      # every route dropped
        meta = orc.sort_metadata(ids, E, block)
        counts, total, rows, eob = _metadata_by_definition_dropping(ids, E, block)
        assert list(meta.counts) == counts
        assert meta.num_post_pad == total
        assert list(meta.sorted_ids) == rows
        assert list(meta.expert_of_block) == eob
        assert orc.check_sort_invariants(ids, meta.sorted_ids, meta.expert_of_block,
                                         meta.num_post_pad, E, block) == []
    ids = np.full((M, k), -1)
    assert orc.sort_metadata(ids, E, block).num_post_pad == 0


def test_checker_rejects_rows_for_dropped_slots():
    ids = np.array([[0, -1], [1, 5]])  # E = 3: slots 1 and 3 are dropped
    meta = orc.sort_metadata(ids, 3, 2)
    assert orc.check_sort_invariants(ids, meta.sorted_ids, meta.expert_of_block, meta.num_post_pad, 3, 2) == []
    bad = meta.sorted_ids.copy()
    bad[1] = 1  # the padding row of expert 0 now claims the dropped slot 1
    assert orc.check_sort_invariants(ids, bad, meta.expert_of_block, meta.num_post_pad, 3, 2) != []


# ---------------------------------------------------------------------------
# The checkers must trip on corrupted metadata (planted mistakes).
# ---------------------------------------------------------------------------
def test_invariant_checker_trips_on_corruption():
    rng = np.random.default_rng(10)
    E, block = 12, 4
    ids = np.stack([np.sort(rng.choice(E, 3, replace=False)) for _ in range(10)])
    m = orc.sort_metadata(ids, E, block)
    good = (m.sorted_ids.copy(), m.expert_of_block.copy(), m.num_post_pad)
    assert orc.check_sort_invariants(ids, *good, E, block) == []
    sentinel = ids.size

    def trips(rows, eob, npp):
        return orc.check_sort_invariants(ids, rows, eob, npp, E, block) != []

    real = np.flatnonzero(good[0] != sentinel)
    rows = good[0].copy(); rows[real[0]], rows[real[1]] = rows[real[1]], rows[real[0]]
    assert trips(rows, good[1], good[2])                      # order inside a segment
    rows = good[0].copy(); rows[real[0]] = rows[real[-1]]
    assert trips(rows, good[1], good[2])                      # duplicated slot
    pad = np.flatnonzero(good[0] == sentinel)
    if pad.size:
        rows = good[0].copy(); rows[pad[0]] = 0
        assert trips(rows, good[1], good[2])                  # padding not sentinel
    eob = good[1].copy(); eob[0] = (eob[0] + 1) % E
    assert trips(good[0], eob, good[2])                       # wrong block owner
    assert trips(good[0], good[1], good[2] - block)           # wrong total


def test_selection_checker_trips():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((4, 24)).astype(np.float32)
    b = np.zeros(24, np.float32)
    res = orc.route_sort(x, "f32", b, 3, 4, 2, 4)
    assert orc.check_selection_invariants(res.keys, res.ids, 4, 2) == []
    bad = res.ids.copy()
    bad[0, 0] = [e for e in range(24) if e not in bad[0]][0]
    bad[0] = np.sort(bad[0])
    assert orc.check_selection_invariants(res.keys, bad, 4, 2) != []


def test_planted_mistakes_are_caught(monkeypatch):
    """A plausible oracle mistake (group score = max instead of top-2 sum, or
    ties to the higher index) must fail the brute-force pin."""
    rng = np.random.default_rng(13)
    keys = [rng.choice(np.array([0.1, 0.4, 0.5, 0.9], np.float32), 12) for _ in range(60)]

    def agree():
        return all(list(orc.route_token(k, 4, 2, 3).ids) == _brute_force_route(k, 4, 2, 3)
                   for k in keys)

    assert agree()
    real_gs = orc.group_scores
    monkeypatch.setattr(orc, "group_scores",
                        lambda key_row, n_group: key_row.reshape(n_group, -1).max(axis=1))
    assert not agree()
    monkeypatch.setattr(orc, "group_scores", real_gs)
    assert agree()
    idx_rank = orc.rank_desc
    monkeypatch.setattr(orc, "rank_desc", lambda v: np.lexsort((-np.arange(v.shape[0]), -v.astype(np.float64))))
    assert not agree()
    monkeypatch.setattr(orc, "rank_desc", idx_rank)


# ---------------------------------------------------------------------------
# Workload generators: deterministic per seed, right shapes.
# ---------------------------------------------------------------------------
def test_workloads_deterministic_and_shaped():
    for name in ["tiny", "decode", "threshold"]:
        cfg = workloads.CONFIGS[name]
        a = workloads.make_inputs(cfg)
        b = workloads.make_inputs(cfg)
        assert a.logits_storage.shape == (cfg.M, cfg.E)
        assert np.array_equal(a.logits_storage, b.logits_storage)
        assert np.array_equal(a.bias, b.bias)
        assert a.bias.dtype == np.float32 and np.all(np.abs(a.bias) <= cfg.bias_range)
        if cfg.dtype == "bf16":
            assert a.logits_storage.dtype == np.uint16
            assert np.array_equal(orc.bf16_bits_to_f32(a.logits_storage), a.logits_f32)


def test_oracle_end_to_end_tiny_invariants():
    cfg = workloads.CONFIGS["tiny"]
    inp = workloads.make_inputs(cfg)
    r = orc.route_sort(inp.logits_storage, cfg.dtype, inp.bias, cfg.k, cfg.n_group,
                       cfg.topk_group, cfg.block)
    assert orc.check_selection_invariants(r.keys, r.ids, cfg.n_group, cfg.topk_group) == []
    assert orc.check_sort_invariants(r.ids, r.meta.sorted_ids, r.meta.expert_of_block,
                                     r.meta.num_post_pad, cfg.E, cfg.block) == []


# ---------------------------------------------------------------------------
# Expert-parallel local metadata
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,E,k,block,ranks", [(50, 64, 4, 8, 4), (7, 12, 3, 1, 3), (200, 896, 16, 128, 8)])
def test_local_metadata_partitions_the_global_metadata(M, E, k, block, ranks):
    # each rank's rows are exactly the global rows of its experts, in the same
    # order, and the ranks' counts add up to the global ones
    rng = np.random.default_rng(M + E)
    ids = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(M)]).astype(np.int32)
    g = orc.sort_metadata(ids, E, block)
    EL = E // ranks
    total = 0
    for r in range(ranks):
        m = orc.local_metadata(ids, r * EL, EL, block)
        assert np.array_equal(m.counts, g.counts[r * EL:(r + 1) * EL])
        lo, hi = g.offsets[r * EL], (g.offsets[(r + 1) * EL] if (r + 1) * EL < E else g.num_post_pad)
        assert np.array_equal(m.sorted_ids, g.sorted_ids[lo:hi])
        assert np.array_equal(m.expert_of_block + r * EL, g.expert_of_block[lo // block:hi // block])
        total += int(m.counts.sum())
    assert total == M * k


def test_local_metadata_small_example():
    # two tokens, k = 2, experts 0..3, the rank owns experts 1 and 2
    ids = np.array([[1, 3], [0, 1]], dtype=np.int32)
    m = orc.local_metadata(ids, 1, 2, 2)
    # expert 1 (local 0) takes slots 0 and 3; expert 2 (local 1) takes none
    assert m.num_post_pad == 2
    assert m.sorted_ids.tolist() == [0, 3]
    assert m.expert_of_block.tolist() == [0]
    full = orc.local_metadata(ids, 0, 4, 2)
    g = orc.sort_metadata(ids, 4, 2)
    assert np.array_equal(full.sorted_ids, g.sorted_ids) and np.array_equal(full.expert_of_block, g.expert_of_block)
