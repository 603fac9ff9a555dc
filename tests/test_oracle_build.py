"""Pins for the draft-tree search oracle.

A tree of T nodes is the sequential best-first result exactly when
  (a) parent[0] = -1 and 0 <= parent[i] < i;
  (b) cum[i] = cum[parent[i]] + log_softmax(row parent[i] / tau)[token[i]];
  (c) ids are in strictly increasing (-cum, parent, token) order;
  (d) every child of a taken node that was not taken scores below node T-1
      (it sorts after it).
Induction on the id: (c) and (d) make node n the best child, not yet taken,
of nodes 0 .. n - 1, which is the search's rule.  The properties are checked
here with scipy's log_softmax and a brute-force scan of every child, not with
the oracle's code.  Plus a two-token closed form and agreement with the input
generator's own best-first tree."""
import numpy as np
import pytest
from scipy.special import log_softmax

import oracle
from synth.inputs import f32_to_bf16_bits, bf16_bits_to_f32


def check_best_first(draft, tau, parent, token, cum, root_token):
    T, V = len(parent), draft.shape[1]
    lp = log_softmax(np.asarray(draft, np.float64)[:T] / tau, axis=1)
    assert parent[0] == -1 and token[0] == root_token and cum[0] == 0.0
    for i in range(1, T):
        assert 0 <= parent[i] < i
        assert cum[i] == pytest.approx(cum[parent[i]] + lp[parent[i], token[i]], abs=1e-12)
    keys = [(-cum[i], int(parent[i]), int(token[i])) for i in range(1, T)]
    assert all(keys[j] < keys[j + 1] for j in range(len(keys) - 1))
    taken = {(int(parent[i]), int(token[i])) for i in range(1, T)}
    assert len(taken) == T - 1
    if T > 1:
        last = keys[-1]
        for e in range(T):
            sc = cum[e] + lp[e]
            for x in range(V):
                if (e, x) not in taken:
                    assert (-sc[x], e, x) > last


@pytest.mark.parametrize("T,V,tau,dt,seed", [(1, 7, 1.0, "f32", 0), (2, 7, 1.0, "f32", 1),
                                             (12, 5, 1.0, "f32", 2), (40, 50, 0.6, "f32", 3),
                                             (40, 50, 1.0, "bf16", 4), (60, 3, 1.3, "f32", 5)])
def test_build_tree_is_best_first(T, V, tau, dt, seed):
    rng = np.random.default_rng(seed)
    d = (rng.standard_normal((T, V)) * 3).astype(np.float32)
    if dt == "bf16":
        stored = f32_to_bf16_bits(d)
        d = bf16_bits_to_f32(stored)
    else:
        stored = d
    parent, token, cum = oracle.build_tree(stored, dt, tau, T, root_token=3 % V)
    check_best_first(d, tau, parent, token, cum, 3 % V)


def test_peaked_rows_give_a_chain():
    """Each row puts almost all mass on one token: the tree is that token's
    chain until the chain's probability falls below the second-best root
    child's."""
    T, V = 30, 16
    d = np.zeros((T, V), np.float32)
    d[:, 4] = 9.0
    parent, token, cum = oracle.build_tree(d, "f32", 1.0, T)
    check_best_first(d, 1.0, parent, token, cum, 0)


def test_two_token_closed_form():
    """Identical rows with p(0) = 0.9, p(1) = 0.1: the chain of k zeros has
    probability 0.9^k, at least 0.1 for k <= 21 (0.9^21 = 0.109, 0.9^22 =
    0.098), and every other continuation is at most 0.1 (the root's child 1)
    or 0.09 (0 then 1).  So 23 nodes are the root, the chain of 21 zeros and
    then the root's child 1."""
    T = 23
    d = np.tile(np.log(np.array([0.9, 0.1])), (T, 1)).astype(np.float64)
    parent, token, cum = oracle.build_tree(d.astype(np.float32), "f32", 1.0, T)
    assert list(parent[:22]) == [-1] + list(range(21))
    assert list(token[1:22]) == [0] * 21
    assert parent[22] == 0 and token[22] == 1
    assert cum[21] == pytest.approx(21 * np.log(0.9), abs=1e-6)


def test_agrees_with_the_input_generator():
    """The 2048-node workload's tree comes from the input generator's own
    best-first search; the oracle builds the same one from the same table."""
    from synth import CONFIGS
    from synth.inputs import _normals, _rng, S_DRAFT, _sssp_tree
    c = CONFIGS["specexec_70b_tree2048"]
    T, V = 300, 2000
    d = _normals(_rng(c, S_DRAFT), (T, V), c.logit_sigma, "f32")
    p_gen, t_gen = _sssp_tree(c, d)
    parent, token, _ = oracle.build_tree(d, "f32", 1.0, T)
    assert np.array_equal(parent, p_gen) and np.array_equal(token[1:], t_gen[1:])
