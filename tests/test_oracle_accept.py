"""Pins for the acceptance oracle: planted greedy prefixes and ties, and
chi-square tests that the emitted tokens follow the target distribution
(with a negative control showing the test has power)."""
import numpy as np
import pytest
from scipy import stats

import oracle


def target_probs(logits, tau):
    """Independent of the oracle's softmax: scipy's."""
    from scipy.special import softmax as sp_softmax
    return sp_softmax(np.asarray(logits, np.float64) / tau)


def _greedy_chain_case(L, T=6, V=50, seed=0):
    """Chain whose first L drafts match the target argmax and whose next one does not."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((1, T, V)).astype(np.float32)
    tokens = np.zeros((1, T), np.int32)
    tokens[0, 0] = 7
    for j in range(T):
        a = (3 * j + 5) % V
        logits[0, j, a] = 10.0                  # argmax of node j's row is a
        if j + 1 < T:
            tokens[0, j + 1] = a if j < L else (a + 1) % V
    return logits, tokens


@pytest.mark.parametrize("L", range(0, 6))
def test_greedy_chain_accepts_longest_matching_prefix(L):
    """Check (c): for a chain the path is the longest prefix whose draft tokens
    equal the target argmax; the bonus is the argmax after it."""
    T = 6
    logits, tokens = _greedy_chain_case(L, T)
    parent = np.arange(-1, T - 1, dtype=np.int32)[None]
    path, plen, bonus = oracle.accept(logits, "f32", None, parent, tokens,
                                      np.zeros((1, T, 2), np.float32), 0.0)
    assert plen[0] == L + 1
    assert list(path[0, :L + 1]) == list(range(L + 1))
    assert np.all(path[0, L + 1:] == -1)
    assert bonus[0] == (3 * L + 5) % 50


def test_greedy_ties_and_duplicate_siblings():
    """Argmax ties go to the lowest token id; duplicate sibling tokens to the
    lowest node index."""
    V = 10
    logits = np.zeros((1, 5, V), np.float32)
    logits[0, 0, [4, 2, 8]] = 3.0                 # tie between 2, 4, 8 -> 2
    logits[0, 2, 6] = 1.0
    parent = np.array([[-1, 0, 0, 0, 2]], np.int32)
    tokens = np.array([[0, 4, 2, 2, 6]], np.int32)  # nodes 2 and 3 both carry token 2
    path, plen, bonus = oracle.accept(logits, "f32", None, parent, tokens,
                                      np.zeros((1, 5, 2), np.float32), 0.0)
    assert list(path[0, :plen[0]]) == [0, 2, 4]
    assert bonus[0] == 0                           # node 4's row is all zeros -> token 0


def _mss_trials(n_trials, n_children, p_logits, q, tau, seed, deterministic=False):
    """n_trials independent steps over a root with n_children i.i.d. draft children
    (or, deterministic=True, the children fixed to q's top tokens)."""
    rng = np.random.default_rng(seed)
    V = len(q)
    T = 1 + n_children
    parent = np.array([[-1] + [0] * n_children], np.int32)
    if deterministic:
        top = np.argsort(-q, kind="stable")[:n_children]
        tokens = np.tile(np.concatenate([[0], top]).astype(np.int32), (n_trials, 1))
    else:
        tokens = np.zeros((n_trials, T), np.int32)
        tokens[:, 1:] = rng.choice(V, size=(n_trials, n_children), p=q)
    logits = np.broadcast_to(np.asarray(p_logits, np.float32), (n_trials, T, V))
    qd = np.broadcast_to(np.asarray(q, np.float32), (n_trials, T, V))
    unif = (rng.integers(0, 1 << 24, size=(n_trials, T, 2)) * 2.0 ** -24).astype(np.float32)
    return logits, qd, parent, tokens, unif


def _first_emitted(path, plen, bonus, tokens):
    return np.where(plen > 1, tokens[np.arange(len(plen)), np.maximum(path[:, 1], 0)], bonus)


P_LOGITS = np.array([1.2, -0.3, 0.4, 2.0, -1.0, 0.0, 0.9, -2.2])
Q_DRAFT = np.array([0.05, 0.30, 0.05, 0.10, 0.25, 0.05, 0.15, 0.05])
N_TRIALS = 200_000


@pytest.mark.parametrize("n_children,n_trials", [(1, N_TRIALS), (2, N_TRIALS), (4, 1_000_000)])
def test_rejection_sampling_emits_target_distribution(n_children, n_trials):
    """Check (d): on a vocabulary of 8 the first emitted token of rejection
    sampling over i.i.d. siblings follows softmax(l / tau) (chi-square p > 0.01),
    10^6 trials for the four-sibling case."""
    tau = 0.8
    logits, qd, parent, tokens, unif = _mss_trials(n_trials, n_children, P_LOGITS, Q_DRAFT, tau,
                                                   seed=10 + n_children)
    path, plen, bonus = oracle.accept(logits, "f32", qd, parent, tokens, unif, tau)
    first = _first_emitted(path, plen, bonus, tokens)
    obs = np.bincount(first, minlength=8)
    exp = target_probs(P_LOGITS, tau) * n_trials
    assert stats.chisquare(obs, exp).pvalue > 0.01


def test_exec_on_deterministic_tree_emits_target_and_mss_does_not():
    """Sampling from the target at each node stays exact on a deterministic
    top-2 tree; rejection sampling on the same fixed tree is biased, and the
    chi-square test detects it (negative control)."""
    tau = 0.6
    logits, qd, parent, tokens, unif = _mss_trials(N_TRIALS, 2, P_LOGITS, Q_DRAFT, tau, seed=21,
                                                   deterministic=True)
    exp = target_probs(P_LOGITS, tau) * N_TRIALS
    path, plen, bonus = oracle.accept(logits, "f32", None, parent, tokens, unif, tau)
    obs = np.bincount(_first_emitted(path, plen, bonus, tokens), minlength=8)
    assert stats.chisquare(obs, exp).pvalue > 0.01
    path, plen, bonus = oracle.accept(logits, "f32", qd, parent, tokens, unif, tau)
    obs = np.bincount(_first_emitted(path, plen, bonus, tokens), minlength=8)
    assert stats.chisquare(obs, exp).pvalue < 1e-6


def test_two_token_joint_on_chains():
    """Joint law of the first two emitted tokens over a two-draft chain: the
    target at node 1 depends on node 1's token through a fixed 8 x 8 table;
    when the step ends early the next token is drawn from that table (what the
    target would do next).  The joint must be p0(t1) * p1(t2 | t1)."""
    tau, V, n = 1.0, 8, N_TRIALS
    rng = np.random.default_rng(33)
    cond = rng.standard_normal((V, V))
    q0 = Q_DRAFT
    q1 = np.roll(Q_DRAFT, 3)
    parent = np.array([[-1, 0, 1]], np.int32)
    tokens = np.zeros((n, 3), np.int32)
    tokens[:, 1] = rng.choice(V, size=n, p=q0)
    tokens[:, 2] = rng.choice(V, size=n, p=q1)
    logits = np.zeros((n, 3, V), np.float32)
    logits[:, 0] = P_LOGITS
    logits[:, 1] = cond[tokens[:, 1]]
    logits[:, 2] = 0.0
    qd = np.zeros((n, 3, V), np.float32)
    qd[:, 0] = q0
    qd[:, 1] = q1
    qd[:, 2] = 1.0 / V
    unif = (rng.integers(0, 1 << 24, size=(n, 3, 2)) * 2.0 ** -24).astype(np.float32)
    path, plen, bonus = oracle.accept(logits, "f32", qd, parent, tokens, unif, tau)
    t1 = np.where(plen > 1, tokens[:, 1], bonus)
    t2 = np.where(plen > 2, tokens[:, 2], np.where(plen == 2, bonus, -1))
    p1 = np.stack([target_probs(cond[a], tau) for a in range(V)])
    nxt = rng.random(n)
    redraw = t2 < 0
    cdf = np.cumsum(p1[t1[redraw]], axis=1)
    t2[redraw] = np.minimum((cdf <= nxt[redraw, None]).sum(axis=1), V - 1)
    obs = np.bincount(t1 * V + t2, minlength=V * V)
    exp = (target_probs(P_LOGITS, tau)[:, None] * p1).ravel() * n
    assert stats.chisquare(obs, exp).pvalue > 0.01


def test_rejection_special_cases():
    """p = q accepts the first child for every uniform; a one-hot draft at x is
    accepted with probability p(x)."""
    tau = 1.0
    p = target_probs(P_LOGITS, tau)
    logits, qd, parent, tokens, unif = _mss_trials(5000, 3, P_LOGITS, p, tau, seed=40)
    path, plen, bonus = oracle.accept(logits, "f32", qd, parent, tokens, unif, tau)
    assert np.all(path[:, 1] == 1)
    x = 6
    onehot = np.zeros(8)
    onehot[x] = 1.0
    logits, qd, parent, tokens, unif = _mss_trials(N_TRIALS, 1, P_LOGITS, onehot, tau, seed=41)
    path, plen, bonus = oracle.accept(logits, "f32", qd, parent, tokens, unif, tau)
    rate = np.mean(plen > 1)
    assert abs(rate - p[x]) < 4 * np.sqrt(p[x] * (1 - p[x]) / N_TRIALS)
    # after the rejection the bonus never repeats x (its residual mass is zero)
    assert np.all(bonus[plen == 1] != x)


def test_invcdf_edges():
    w = np.array([0.0, 0.25, 0.0, 0.75, 0.0])
    assert oracle.invcdf(w, 0.0)[0] == 1
    assert oracle.invcdf(w, 0.2499)[0] == 1
    assert oracle.invcdf(w, 0.25)[0] == 3
    assert oracle.invcdf(w, 0.9999999)[0] == 3


def _one_node_case(V, tokens, q_row, u_test, u_root_sample, u_leaf_sample=0.0):
    """A root whose children carry `tokens` (child c is node c + 1), uniform
    target logits (p = 1/V), the same draft row at every node."""
    n = len(tokens)
    T = n + 1
    parent = np.array([[-1] + [0] * n], np.int32)
    tok = np.array([[0] + list(tokens)], np.int32)
    logits = np.zeros((1, T, V), np.float32)
    qd = np.broadcast_to(np.asarray(q_row, np.float32), (1, T, V)).copy()
    unif = np.zeros((1, T, 2), np.float32)
    unif[0, 1:, 0] = u_test
    unif[0, 0, 1] = u_root_sample
    unif[0, 1:, 1] = u_leaf_sample
    return logits, qd, parent, tok, unif


def test_zero_residual_mass_leaves_target_unchanged():
    """Reading R9: a draft row with q >= p everywhere (here q = 2p, summing to
    2) leaves no residual mass after a rejection; the target is then kept as it
    was.  With p = 1/8, child c is accepted iff u_c * 1/4 < 1/8, i.e. u_c < 1/2,
    whatever came before -- so the walk takes the first child with u < 1/2.
    (Setting r to the zero vector instead would reject every later child; a
    division by the zero mass would turn r into NaNs and reject them too.)"""
    V = 8
    q = np.full(V, 0.25)
    # children 1, 2 rejected (u >= 1/2), child 3 accepted (u = 0.3)
    logits, qd, parent, tok, unif = _one_node_case(V, [3, 5, 1], q, [0.7, 0.6, 0.3], 0.0,
                                                   u_leaf_sample=0.55)
    path, plen, bonus = oracle.accept(logits, "f32", qd, parent, tok, unif, 1.0)
    assert list(path[0, :plen[0]]) == [0, 3]
    # node 3 is a leaf: the bonus is drawn from p = 1/8 there: smallest x with (x+1)/8 > 0.55
    assert bonus[0] == 4
    # every child rejected: the bonus comes from the unchanged target, x = floor(8 u)
    logits, qd, parent, tok, unif = _one_node_case(V, [3, 5, 1], q, [0.7, 0.6, 0.9], 0.8)
    path, plen, bonus = oracle.accept(logits, "f32", qd, parent, tok, unif, 1.0)
    assert plen[0] == 1 and bonus[0] == 6


def test_wide_node_tests_every_sibling():
    """A node with 100 children: the first 99 carry token 0, the last token 3.
    With p = 1/8 and q(0) = 0.9, q(y) = 0.1/7 elsewhere, child 1 is rejected
    (u q(0) = 0.45 >= 1/8); the residual is then uniform over tokens 1..7
    (max(p - q, 0) is the same there and zero at token 0) and stays so after
    every later rejection, while r(0) = 0 rejects children 2..99 for any u.
    Child 100 (token 3, u = 0.9) passes 0.9 * 0.1/7 < 1/7: the path is
    [0, 100], and its leaf draws the bonus from p = 1/8."""
    V = 8
    q = np.full(V, 0.1 / 7)
    q[0] = 0.9
    tokens = [0] * 99 + [3]
    u = [0.5] + [0.99] * 98 + [0.9]
    logits, qd, parent, tok, unif = _one_node_case(V, tokens, q, u, 0.0, u_leaf_sample=0.3)
    path, plen, bonus = oracle.accept(logits, "f32", qd, parent, tok, unif, 1.0)
    assert list(path[0, :plen[0]]) == [0, 100]
    assert bonus[0] == 2                      # smallest x with (x+1)/8 > 0.3
    # the last child made to fail too (u = 0.9999 -> 0.9999 * q(3) < 1/7 still
    # holds, so give it token 0): every child rejected, the bonus is drawn from
    # the residual, uniform over 1..7: smallest x >= 1 with x/7 > 0.5 -> 4
    tokens = [0] * 100
    logits, qd, parent, tok, unif = _one_node_case(V, tokens, q, u, 0.5)
    path, plen, bonus = oracle.accept(logits, "f32", qd, parent, tok, unif, 1.0)
    assert plen[0] == 1 and bonus[0] == 4
