"""Pins of the gate-projection oracle (oracle/gate.py): integer dot products,
selection weights, a rounding midpoint that only exact arithmetic settles, and
agreement with a float64 matrix product within that product's error bound."""
import numpy as np
import pytest

from oracle import gate as og
from workloads import f32_to_bf16_bits


def _bits(a):
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def test_integer_inputs_give_integer_logits():
    rng = np.random.default_rng(0)
    M, E, H = 3, 7, 40
    h = rng.integers(-9, 10, size=(M, H))
    w = rng.integers(-9, 10, size=(E, H))
    got = og.gate_logits(_bits(h), _bits(w))
    assert np.array_equal(got, (h @ w.T).astype(np.float32))


def test_selection_weights_pick_hidden_entries():
    # W[e] is the unit vector at index (5e + 1) mod H
    rng = np.random.default_rng(1)
    M, E, H = 2, 9, 16
    hb = _bits(rng.standard_normal((M, H)))
    w = np.zeros((E, H), dtype=np.float32)
    for e in range(E):
        w[e, (5 * e + 1) % H] = 1.0
    got = og.gate_logits(hb, _bits(w))
    hf = og.bf16_to_f64(hb).astype(np.float32)
    for e in range(E):
        assert np.array_equal(got[:, e], hf[:, (5 * e + 1) % H])


def test_midpoint_is_settled_by_the_exact_sum():
    # 1 + 2^-24 is halfway between the FP32 neighbours 1 and 1 + 2^-23; a
    # further 2^-70 (lost in a float64 sum) decides the rounding upwards, and
    # -2^-70 downwards; without it the tie goes to the even value 1
    for tail, want in ((2.0 ** -70, 1.0 + 2.0 ** -23), (-(2.0 ** -70), 1.0), (0.0, 1.0)):
        h = np.array([[1.0, 2.0 ** -24, tail if tail else 1.0]])
        w = np.array([[1.0, 1.0, 1.0 if tail else 0.0]])
        got = og.gate_logits(_bits(h), _bits(w))
        assert got[0, 0] == np.float32(want), (tail, got[0, 0])
    # the same on the negative side
    got = og.gate_logits(_bits([[-1.0, -(2.0 ** -24), -(2.0 ** -70)]]), _bits([[1.0, 1.0, 1.0]]))
    assert got[0, 0] == np.float32(-(1.0 + 2.0 ** -23))


@pytest.mark.parametrize("seed", [0, 1])
def test_matches_float64_product_within_its_bound(seed):
    rng = np.random.default_rng(seed)
    M, E, H = 2, 32, 7168
    hb = _bits(rng.standard_normal((M, H)))
    wb = _bits(rng.standard_normal((E, H)) * H ** -0.5)
    got = og.gate_logits(hb, wb).astype(np.float64)
    h, w = og.bf16_to_f64(hb), og.bf16_to_f64(wb)
    ref = h @ w.T
    bound = H * 2.0 ** -53 * (np.abs(h) @ np.abs(w).T) + 2.0 ** -24 * np.abs(ref)
    assert np.all(np.abs(got - ref) <= bound)


def test_midpoint_margin_of_a_constructed_tie():
    # exact value 1 + 2^-24 + 2^-70: distance 2^-70 from the midpoint 1 + 2^-24
    h = _bits([[1.0, 2.0 ** -24, 2.0 ** -70]])
    w = _bits([[1.0, 1.0, 1.0]])
    m = og.midpoint_margin(h, w, og.gate_logits(h, w))
    assert m[0, 0] < 2.0 ** -60
    # a value far from any midpoint: 1 + 2^-25 sits a quarter ulp from both
    h2 = _bits([[1.0, 2.0 ** -25]])
    m2 = og.midpoint_margin(h2, _bits([[1.0, 1.0]]), og.gate_logits(h2, _bits([[1.0, 1.0]])))
    assert abs(m2[0, 0] * (1.0 + 2.0 ** -25) - 2.0 ** -25) < 2.0 ** -50
