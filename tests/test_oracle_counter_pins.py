"""Pins for the oracle's sort with caller-provided initial counters (CPU only).

`sort_metadata_counters` follows the page "gfx1250 ordinary-TP route
optimization" (Dispatch and contracts: caller-provided counters keep their
initial offsets; negative ids claim no slot).  Its reading: counter[e] rows
already sit at the head of expert e's segment and this call's routes follow
them.  The pins tie it to the plain sort by two routes that do not share its
code path: zero counters reduce to `sort_metadata`, and counters equal to the
counts of a first batch reproduce the plain sort of both batches
concatenated (the first batch's rows being the untouched ones), plus a
hand-worked example.
"""
import numpy as np
import pytest

from oracle import route_sort as orc


def _ids(rng, M, E, k, drop=0.0):
    ids = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(M)]).astype(np.int32)
    if drop:
        ids[rng.random(ids.shape) < drop] = -1
    return ids


@pytest.mark.parametrize("M,E,k,block", [(5, 8, 3, 4), (40, 64, 4, 16), (33, 100, 6, 1), (200, 896, 16, 128)])
def test_zero_counters_reduce_to_plain_sort(M, E, k, block):
    rng = np.random.default_rng(M + E)
    ids = _ids(rng, M, E, k, drop=0.1)
    cm = orc.sort_metadata_counters(ids, E, block, np.zeros(E, np.int64))
    m = orc.sort_metadata(ids, E, block)
    assert cm.written.all()
    assert cm.meta.num_post_pad == m.num_post_pad
    assert np.array_equal(cm.meta.sorted_ids, m.sorted_ids)
    assert np.array_equal(cm.meta.expert_of_block, m.expert_of_block)
    assert np.array_equal(cm.counters_out, m.counts)


@pytest.mark.parametrize("MA,MB,E,k,block", [(3, 4, 8, 3, 4), (30, 50, 64, 4, 16), (17, 9, 100, 6, 1),
                                             (100, 150, 896, 16, 128), (0, 20, 32, 2, 8), (20, 0, 32, 2, 8)])
def test_counters_of_a_first_batch_match_the_concatenated_sort(MA, MB, E, k, block):
    rng = np.random.default_rng(MA * 7 + MB)
    A = _ids(rng, MA, E, k, drop=0.1) if MA else np.zeros((0, k), np.int32)
    B = _ids(rng, MB, E, k, drop=0.1) if MB else np.zeros((0, k), np.int32)
    both = orc.sort_metadata(np.concatenate([A, B]), E, block)
    c0 = np.bincount(A[(A >= 0) & (A < E)].reshape(-1), minlength=E)
    cm = orc.sort_metadata_counters(B, E, block, c0)
    assert cm.meta.num_post_pad == both.num_post_pad
    assert np.array_equal(cm.meta.offsets, both.offsets)
    assert np.array_equal(cm.meta.expert_of_block, both.expert_of_block)
    assert np.array_equal(cm.counters_out, both.counts)
    rows_b = cm.meta.sorted_ids.astype(np.int64)
    rows_ab = both.sorted_ids.astype(np.int64)
    # untouched rows are exactly the rows of batch A's slots
    assert np.array_equal(~cm.written, rows_ab < MA * k)
    # B's slots, renumbered past A, and the sentinel of the whole
    w = cm.written
    sent_b = rows_b[w] == MB * k
    assert np.array_equal(sent_b, rows_ab[w] == (MA + MB) * k)
    assert np.array_equal(rows_b[w][~sent_b] + MA * k, rows_ab[w][~sent_b])


def test_counters_hand_worked():
    # two tokens, k = 2, experts 0..2, block 2; the caller holds 1 row of expert 0
    # and 2 of expert 2.  Routes: slot 0 -> e0, 1 -> e2, 2 -> e0, 3 -> dropped.
    ids = np.array([[0, 2], [0, -1]], np.int32)
    cm = orc.sort_metadata_counters(ids, 3, 2, np.array([1, 0, 2]))
    # expert 0: 1 + 2 = 3 rows -> 4; expert 1: 0; expert 2: 2 + 1 = 3 -> 4
    assert cm.meta.num_post_pad == 8
    assert cm.meta.offsets.tolist() == [0, 4, 4]
    assert cm.meta.sorted_ids.tolist() == [-1, 0, 2, 4, -1, -1, 1, 4]
    assert cm.written.tolist() == [False, True, True, True, False, False, True, True]
    assert cm.meta.expert_of_block.tolist() == [0, 0, 2, 2]
    assert cm.counters_out.tolist() == [3, 0, 3]
