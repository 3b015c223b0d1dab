"""Pins for the oracle's near-tie gaps (CPU only).

The target asks for tokens whose k-th and (k+1)-th scores differ by less than
1e-6 to be reported separately.  The oracle's `route_token` returns two gaps:

  gap_k = key of the k-th pick - key of the best unpicked expert, both among
          the experts of the kept groups (biased keys, ties broken to the lower
          expert index as the selection breaks them);
  gap_g = score of the weakest kept group - score of the strongest dropped
          group (None when every group is kept).

These tests tie them to something other than the oracle's own sort: exact
binary-fraction examples worked by hand, and a brute-force characterisation
(the k-th largest is the smallest picked key, the (k+1)-th is the largest key
left over among the allowed experts) checked on enumerated tiny shapes.  A
final test plants each plausible mistake (a gap over every expert, the
unbiased score instead of the key, an index off by one) and checks that a pin
trips.
"""
import itertools

import numpy as np
import pytest

from oracle import route_sort as orc


def _gaps_by_brute_force(key: np.ndarray, n_group: int, topk_group: int, k: int):
    """Enumerate every group subset and every expert subset (as the selection
    pin does), then read the gaps off the winning sets by min/max only."""
    E = key.shape[0]
    G = E // n_group
    gs = []
    for g in range(n_group):
        mem = range(g * G, (g + 1) * G)
        gs.append(np.float32(key[g * G]) if G == 1 else
                  max(np.float32(key[i] + key[j]) for i, j in itertools.combinations(mem, 2)))

    def best_subset(items, m, val):
        best, best_sig = None, None
        for sub in itertools.combinations(items, m):
            sig = sorted(((float(val(i)), -i) for i in sub), reverse=True)
            if best_sig is None or sig > best_sig:
                best, best_sig = sub, sig
        return list(best)

    kept = best_subset(range(n_group), topk_group, lambda g: gs[g])
    dropped = [g for g in range(n_group) if g not in kept]
    gap_g = None
    if dropped:
        gap_g = min(float(gs[g]) for g in kept) - max(float(gs[g]) for g in dropped)
    allowed = [e for g in kept for e in range(g * G, (g + 1) * G)]
    picked = best_subset(allowed, k, lambda e: key[e])
    rest = [e for e in allowed if e not in picked]
    gap_k = None
    if rest:
        gap_k = min(float(key[e]) for e in picked) - max(float(key[e]) for e in rest)
    return gap_k, gap_g


# Two groups of four experts; keys are binary fractions, so every key, group
# score and gap below is exact.  Group 0 holds the single best key (0.875) but
# scores 0.875 + 0.25 = 1.125; group 1 scores 0.75 + 0.6875 = 1.4375 and is the
# one kept.  Inside group 1 the order is 0.75 (e5), 0.6875 (e6), 0.5 (e4),
# 0.25 (e7).
HAND_KEYS = np.array([0.875, 0.25, 0.125, 0.0, 0.5, 0.75, 0.6875, 0.25], np.float32)


def test_gap_hand_worked_k2():
    r = orc.route_token(HAND_KEYS, 2, 1, 2)
    assert list(r.ids) == [5, 6]
    assert r.gap_k == 0.6875 - 0.5    # 0.1875; over every expert it would be 0.6875 - 0.875 < 0
    assert r.gap_g == 1.4375 - 1.125  # 0.3125


def test_gap_hand_worked_other_k():
    # off-by-one readings give 0.0625 (k-1 vs k) or 0.25 (k+1 vs k+2) here
    r1 = orc.route_token(HAND_KEYS, 2, 1, 1)
    assert r1.gap_k == 0.75 - 0.6875
    r3 = orc.route_token(HAND_KEYS, 2, 1, 3)
    assert r3.gap_k == 0.5 - 0.25
    # every allowed expert picked: no (k+1)-th key, no gap
    assert orc.route_token(HAND_KEYS, 2, 1, 4).gap_k is None
    # every group kept: no group gap; the expert gap is then over all experts
    r = orc.route_token(HAND_KEYS, 2, 2, 2)
    assert r.gap_g is None
    assert r.gap_k == 0.75 - 0.6875


def test_gap_uses_biased_keys_not_scores():
    # logits 0 give s = 1/2 for every expert, so gaps of the unbiased scores
    # would all be 0; the keys 1/2 + bias reproduce HAND_KEYS exactly
    x = np.zeros((1, 8), np.float32)
    bias = (HAND_KEYS - np.float32(0.5)).astype(np.float32)
    res = orc.route_sort(x, "f32", bias, 2, 2, 1, 4)
    assert np.array_equal(res.keys[0], HAND_KEYS)
    assert res.gap_k[0] == 0.1875
    assert res.gap_g[0] == 0.3125


def test_gap_exact_ties_are_zero():
    key = np.array([0.5, 0.5, 0.25, 0.25, 0.5, 0.5, 0.25, 0.25], np.float32)
    r = orc.route_token(key, 2, 1, 1)
    assert list(r.groups) == [0] and list(r.ids) == [0]
    assert r.gap_k == 0.0 and r.gap_g == 0.0
    # the whole-path arrays carry inf where a gap is undefined
    res = orc.route_sort(np.zeros((1, 4), np.float32), "f32", np.zeros(4, np.float32), 4, 1, 1, 2)
    assert np.isinf(res.gap_k[0]) and np.isinf(res.gap_g[0])


SHAPES = [(6, 3, 2, 2), (8, 4, 2, 3), (8, 2, 1, 4), (9, 3, 1, 2), (10, 5, 3, 4),
          (12, 4, 2, 3), (12, 6, 4, 4), (12, 12, 5, 3), (12, 3, 3, 5), (8, 1, 1, 3)]


def _key_rows(E, seed, n=30):
    rng = np.random.default_rng(seed)
    rows = []
    for t in range(n):
        if t % 3 == 0:
            rows.append(rng.choice(np.array([0.25, 0.5, 0.75], np.float32), E))
        else:
            x = rng.standard_normal(E).astype(np.float32)
            b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
            rows.append(orc.biased_keys(x, b)[1])
    return rows


@pytest.mark.parametrize("E,n_group,topk_group,k", SHAPES)
def test_gap_brute_force(E, n_group, topk_group, k):
    for key in _key_rows(E, E * 31 + n_group * 7 + k):
        r = orc.route_token(key, n_group, topk_group, k)
        gk, gg = _gaps_by_brute_force(key, n_group, topk_group, k)
        assert r.gap_k == gk and r.gap_g == gg, (key, r, gk, gg)


def test_gap_best_unpicked_expert_in_dropped_group():
    # built so that the strongest key outside the picks sits in a dropped group
    # on every row: the gap must ignore it
    rng = np.random.default_rng(99)
    hits = 0
    for _ in range(200):
        key = rng.standard_normal(12).astype(np.float32)
        r = orc.route_token(key, 4, 2, 3)
        allowed = [e for g in r.groups for e in range(3 * g, 3 * g + 3)]
        outside = [e for e in range(12) if e not in allowed]
        if max(key[outside]) > min(key[r.ids]):
            hits += 1
            gk, _ = _gaps_by_brute_force(key, 4, 2, 3)
            assert r.gap_k == gk and r.gap_k > 0
    assert hits > 20


def _mutant(kind):
    real = orc.route_token

    def route_token(key_row, n_group, topk_group, k):
        r = real(key_row, n_group, topk_group, k)
        E = key_row.shape[0]
        if kind == "all_experts":
            order = orc.rank_desc(key_row)
            gap_k = float(key_row[order[k - 1]]) - float(key_row[order[k]]) if E > k else None
        elif kind == "off_by_one":
            G = E // n_group
            allowed = np.concatenate([np.arange(g * G, (g + 1) * G) for g in r.groups])
            order = allowed[orc.rank_desc(key_row[allowed])]
            gap_k = (float(key_row[order[k]]) - float(key_row[order[k + 1]])
                     if allowed.shape[0] > k + 1 else None)
        else:
            gap_k = r.gap_k
        return orc.TokenRoute(r.ids, r.groups, gap_k, r.gap_g)
    return route_token


@pytest.mark.parametrize("kind", ["all_experts", "off_by_one"])
def test_planted_gap_mistakes_are_caught(monkeypatch, kind):
    monkeypatch.setattr(orc, "route_token", _mutant(kind))
    caught = False
    try:
        test_gap_hand_worked_k2()
        test_gap_brute_force(12, 4, 2, 3)
    except AssertionError:
        caught = True
    assert caught


def test_planted_unbiased_gap_is_caught(monkeypatch):
    # a mutant that ranks by the unbiased score when it builds the gaps
    real = orc.biased_keys
    monkeypatch.setattr(orc, "biased_keys", lambda x, b: (real(x, b)[0], real(x, b)[0]))
    with pytest.raises(AssertionError):
        test_gap_uses_biased_keys_not_scores()
