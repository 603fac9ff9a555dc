"""Pins for the draft-tree expansion step: closed forms, a monotone special
case, normalisation, and the temperature identity."""
import math

import numpy as np

import oracle
from synth.inputs import f32_to_bf16_bits


def test_uniform_logits_closed_form():
    """Equal logits: every candidate of row e scores cum[e] - log V, so the
    best are the rows by cumulative log-probability, tokens ascending."""
    E, V, k = 3, 5, 7
    cum = np.array([-1.0, -0.25, -2.0], np.float32)
    row, tok, sc = oracle.expand(np.zeros((E, V), np.float32), "f32", cum, 1.0, k)
    assert row.tolist() == [1] * 5 + [0] * 2
    assert tok.tolist() == [0, 1, 2, 3, 4, 0, 1]
    assert np.allclose(sc, [-0.25 - math.log(5)] * 5 + [-1.0 - math.log(5)] * 2, rtol=0, atol=1e-12)


def test_single_row_keeps_largest_logits():
    """One row: the kept tokens are the k largest logits, ties by token."""
    rng = np.random.default_rng(1)
    l = rng.integers(-4, 5, size=(1, 40)).astype(np.float32)       # many exact ties
    row, tok, _ = oracle.expand(l, "f32", np.zeros(1, np.float32), 0.7, 12)
    want = sorted(range(40), key=lambda x: (-l[0, x], x))[:12]
    assert tok.tolist() == want and (row == 0).all()


def test_known_probabilities():
    """Logits (0, log 3) at temperature 1: probabilities 1/4 and 3/4."""
    l = np.array([[0.0, math.log(3.0)]], np.float64).astype(np.float32)
    _, tok, sc = oracle.expand(l, "f32", np.array([0.5], np.float32), 1.0, 2)
    assert tok.tolist() == [1, 0]
    assert abs(sc[0] - (0.5 + math.log(0.75))) < 1e-7 and abs(sc[1] - (0.5 + math.log(0.25))) < 1e-7


def test_rows_normalise_and_temperature_identity():
    rng = np.random.default_rng(2)
    E, V = 4, 33
    l = (rng.standard_normal((E, V)) * 3).astype(np.float32)
    cum = (-rng.random(E)).astype(np.float32)
    row, tok, sc = oracle.expand(l, "f32", cum, 0.6, E * V)
    # all candidates returned: each row's probabilities sum to one
    for e in range(E):
        p = np.exp(sc[row == e] - np.float64(cum[e]))
        assert abs(p.sum() - 1.0) < 1e-12
    # scores are non-increasing and ties go to the smaller (e, x)
    flat = row.astype(np.int64) * V + tok
    assert all(sc[i] > sc[i + 1] or (sc[i] == sc[i + 1] and flat[i] < flat[i + 1]) for i in range(len(sc) - 1))
    # logits scaled by tau at temperature tau are the logits at temperature 1
    l2 = np.float32(2.0) * l                        # exact in float32
    a = oracle.expand(l, "f32", cum, 1.0, 20)
    b = oracle.expand(l2, "f32", cum, 2.0, 20)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and np.allclose(a[2], b[2], atol=1e-12)


def test_bf16_rows_decode():
    rng = np.random.default_rng(3)
    l = (rng.standard_normal((2, 16)) * 2).astype(np.float32)
    bits = f32_to_bf16_bits(l)
    a = oracle.expand(bits, "bf16", np.zeros(2, np.float32), 1.0, 5)
    b = oracle.expand(np.asarray(oracle.decode(bits, "bf16"), np.float32), "f32", np.zeros(2, np.float32), 1.0, 5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
