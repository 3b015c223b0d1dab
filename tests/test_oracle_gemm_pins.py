"""Pins of the grouped-GEMM oracle (oracle/moe_gemm.py) to facts that do not
come from the oracle itself: integer arithmetic, closed forms, the metadata's
own meaning (each token slot's pick), and the rounding bound the tolerance
rests on."""
import numpy as np
import pytest

from oracle import moe_gemm as og
from oracle import route_sort as ors
from workloads import f32_to_bf16_bits


def _ids(rng, M, E, k):
    """Distinct experts per token, as a router returns them."""
    return np.stack([np.sort(rng.choice(E, size=k, replace=False)) for _ in range(M)]).astype(np.int32)


def _meta(ids, E, block):
    m = ors.sort_metadata(ids, E, block)
    return m.sorted_ids, m.expert_of_block, m.num_post_pad


def _bits(a):
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


@pytest.mark.parametrize("M,E,k,K,N,block", [(7, 5, 2, 24, 8, 4), (33, 12, 3, 40, 16, 8), (1, 6, 4, 16, 4, 32)])
def test_integer_inputs_match_dense_integer_product(M, E, k, K, N, block):
    # small integers are exact in BF16 and their products and sums are exact
    # in float64, so every output must equal the integer product for the
    # expert that the token slot picked
    rng = np.random.default_rng(M * 100 + E)
    xi = rng.integers(-8, 9, size=(M, K)).astype(np.int64)
    wi = rng.integers(-8, 9, size=(E, N, K)).astype(np.int64)
    dense = np.einsum("tk,enk->ten", xi, wi)  # [M, E, N]
    ids = _ids(rng, M, E, k)
    sid, eob, npp = _meta(ids, E, block)
    y = og.gemm1_sorted(_bits(xi), _bits(wi), sid, eob, npp, M, k, block)
    assert y.shape == (npp, N)
    seen = np.zeros(npp, dtype=bool)
    for t in range(M):
        for j in range(k):
            (r,) = np.nonzero(sid == t * k + j)[0]
            assert np.array_equal(y[r], dense[t, ids[t, j]].astype(np.float64))
            seen[r] = True
    # every other row is padding and holds zeros
    assert np.all(y[~seen] == 0)
    assert np.all(sid[~seen] == M * k)


def test_selection_weights_give_shifted_columns():
    # W[e][n, i] = 1 exactly when i == (n + 3e) mod K, so y[r, n] = x[t, (n + 3e) mod K]
    rng = np.random.default_rng(5)
    M, E, k, K, N, block = 9, 6, 2, 32, 16, 4
    x = rng.standard_normal((M, K)).astype(np.float32)
    xb = _bits(x)
    w = np.zeros((E, N, K), dtype=np.float32)
    for e in range(E):
        for n in range(N):
            w[e, n, (n + 3 * e) % K] = 1.0
    ids = _ids(rng, M, E, k)
    sid, eob, npp = _meta(ids, E, block)
    y = og.gemm1_sorted(xb, _bits(w), sid, eob, npp, M, k, block)
    xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for t in range(M):
        for j in range(k):
            (r,) = np.nonzero(sid == t * k + j)[0]
            e = ids[t, j]
            assert np.array_equal(y[r], xf[t, (np.arange(N) + 3 * e) % K])


def test_constant_matrices_give_closed_form():
    # x[t, :] = t + 1 and W[e] = (e + 1) everywhere: y = K (t + 1)(e + 1)
    M, E, k, K, N, block = 6, 4, 2, 64, 8, 2
    x = np.repeat(np.arange(1, M + 1, dtype=np.float32)[:, None], K, axis=1)
    w = np.repeat(np.arange(1, E + 1, dtype=np.float32)[:, None, None], N, axis=1).repeat(K, axis=2)
    ids = np.array([[t % E, (t + 1) % E] for t in range(M)], dtype=np.int32)
    ids.sort(axis=1)
    sid, eob, npp = _meta(ids, E, block)
    y = og.gemm1_sorted(_bits(x), _bits(w), sid, eob, npp, M, k, block)
    for r in range(npp):
        s = sid[r]
        if s == M * k:
            assert np.all(y[r] == 0)
        else:
            t, e = s // k, eob[r // block]
            assert e == ids[t, s % k]
            assert np.all(y[r] == K * (t + 1) * (e + 1))


def test_sampled_rows_equal_full_result_and_sentinels_are_zero():
    rng = np.random.default_rng(11)
    M, E, k, K, N, block = 40, 10, 4, 48, 12, 8
    xb = _bits(rng.standard_normal((M, K)))
    wb = _bits(rng.standard_normal((E, N, K)) * 0.05)
    ids = _ids(rng, M, E, k)
    sid, eob, npp = _meta(ids, E, block)
    full = og.gemm1_sorted(xb, wb, sid, eob, npp, M, k, block)
    rows = rng.choice(npp, size=25, replace=False)
    assert np.array_equal(og.gemm1_rows(xb, wb, sid, eob, M, k, block, rows), full[rows])
    assert np.all(full[sid == M * k] == 0)


def test_dropped_slots_are_padding():
    # a negative or out-of-range slot value in sorted_ids never reads x
    M, E, k, K, N, block = 3, 2, 1, 16, 4, 2
    xb = _bits(np.ones((M, K)))
    wb = _bits(np.ones((E, N, K)))
    sid = np.array([0, -1, 2, 3, 99, 1], dtype=np.int32)   # 3 == M*k: sentinel
    eob = np.array([0, 1, 1], dtype=np.int32)
    y = og.gemm1_sorted(xb, wb, sid, eob, 6, M, k, block)
    assert np.all(y[[1, 3, 4]] == 0)
    assert np.all(y[[0, 2, 5]] == K)


def test_bf16_rounding_is_nearest_even():
    # every BF16 value converts to itself; halfway points go to the even pattern
    pats = np.arange(0, 0x10000, dtype=np.uint32)
    pats = pats[((pats >> 7) & 0xFF) != 0xFF]  # finite values only
    vals = (pats << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(og.f64_to_bf16_bits(vals), pats.astype(np.uint16))
    lo = np.float32(1.0)
    mid = np.float64(1.0 + 2.0 ** -8)        # halfway between 1 and 1 + 2^-7
    assert og.f64_to_bf16_bits(np.array([mid]))[0] == (np.array([lo]).view(np.uint32)[0] >> 16)
    mid2 = np.float64(1.0 + 3 * 2.0 ** -8)   # halfway between 1 + 2^-7 and 1 + 2^-6
    assert og.f64_to_bf16_bits(np.array([mid2]))[0] == 0x3F82


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tolerance_covers_fp32_accumulation_in_any_order(seed):
    # an FP32 running sum of the exact products in a random order, rounded to
    # BF16, stays within the tolerance of the exact value
    rng = np.random.default_rng(seed)
    K, n = 3584, 64
    x = rng.standard_normal((n, K)).astype(np.float32)
    w = (rng.standard_normal((n, K)) * 0.02).astype(np.float32)
    xb, wb = _bits(x), _bits(w)
    xf = og.bf16_to_f64(xb)
    wf = og.bf16_to_f64(wb)
    prod = xf * wf
    exact = prod.sum(axis=1)
    absp = np.abs(prod).sum(axis=1)
    got = np.empty(n)
    for i in range(n):
        p = prod[i, rng.permutation(K)].astype(np.float32)
        acc = np.float32(0)
        for v in p:
            acc = np.float32(acc + v)
        got[i] = og.bf16_to_f64(og.f64_to_bf16_bits(np.array([acc], dtype=np.float64)))[0]
    tol = og.tolerance(exact, absp, K)
    assert np.all(np.abs(got - exact) <= tol)
    # and the bound is not vacuous: it is far below the size of the values
    assert np.median(tol / np.maximum(np.abs(exact), 1e-30)) < 0.05
