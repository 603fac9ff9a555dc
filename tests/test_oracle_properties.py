"""Property tests of the oracle over random small trees, shapes and shuffled
block tables (hypothesis-generated, seeded by hypothesis's own database):
invariants that hold for any input.

* attention: the all-nodes formulation equals the per-root-path causal one;
  the output is invariant under a reshuffle of the physical blocks (same
  logical cache, another block table); a node's output does not depend on
  the keys of nodes that are not its ancestors.
* greedy acceptance: the path is a root path of the tree, each accepted
  node's token is the argmax of its parent's row, and the bonus is the
  argmax of the last node's row, no child of which carries it.
* commit: the committed context read back through the table is the old
  context followed by the accepted path's rows; nothing else changes.
"""
import numpy as np
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
from tests.helpers import paged_from_dense

SETTINGS = dict(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def tree_case(draw, max_T=9):
    T = draw(st.integers(1, max_T))
    parent = [-1] + [draw(st.integers(0, i - 1)) for i in range(1, T)]
    B = draw(st.integers(1, 3))
    Hkv = draw(st.sampled_from([1, 2]))
    G = draw(st.sampled_from([1, 2, 3]))
    D = draw(st.sampled_from([4, 8]))
    bs = draw(st.sampled_from([2, 3, 4, 8]))
    ctx = [draw(st.integers(0, 20)) for _ in range(B)]
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return np.array(parent, np.int32), B, Hkv, G, D, bs, ctx, seed


def _cache(B, Hkv, G, D, bs, ctx, T, seed, shuffle_seed=None):
    rng = np.random.default_rng(seed)
    n = max(ctx) + T
    Kd = rng.standard_normal((B, Hkv, n, D))
    Vd = rng.standard_normal((B, Hkv, n, D))
    q = rng.standard_normal((B, T, Hkv * G, D))
    srng = None if shuffle_seed is None else np.random.default_rng(shuffle_seed)
    kp, vp, table = paged_from_dense(Kd, Vd, bs, srng, spare=1)
    return q, kp, vp, table, np.array(ctx, np.int32), Kd, Vd


@settings(**SETTINGS)
@given(tree_case())
def test_attention_formulations_agree_and_ignore_the_table(case):
    parent, B, Hkv, G, D, bs, ctx, seed = case
    T = len(parent)
    tp = np.tile(parent, (B, 1))
    q, kp, vp, table, cl, Kd, Vd = _cache(B, Hkv, G, D, bs, ctx, T, seed)
    a = oracle.attention_dense(q, kp, vp, table, cl, tp, bs, "f32")
    b = oracle.attention_by_path(q, kp, vp, table, cl, tp, bs, "f32")
    assert np.max(np.abs(a - b)) < 1e-12
    q2, kp2, vp2, table2, _, _, _ = _cache(B, Hkv, G, D, bs, ctx, T, seed, shuffle_seed=seed + 1)
    c = oracle.attention_dense(q2, kp2, vp2, table2, cl, tp, bs, "f32")
    assert np.max(np.abs(a - c)) < 1e-12


@settings(**SETTINGS)
@given(tree_case(), st.integers(0, 2 ** 31 - 1))
def test_attention_ignores_non_ancestor_keys(case, seed2):
    parent, B, Hkv, G, D, bs, ctx, seed = case
    T = len(parent)
    tp = np.tile(parent, (B, 1))
    q, kp, vp, table, cl, Kd, Vd = _cache(B, Hkv, G, D, bs, ctx, T, seed)
    a = oracle.attention_dense(q, kp, vp, table, cl, tp, bs, "f32")
    anc = oracle.ancestor_matrix(parent)
    i = int(np.random.default_rng(seed2).integers(T))
    # scramble every tree slot that is not an ancestor of node i
    kp2, vp2 = kp.copy(), vp.copy()
    r = np.random.default_rng(seed2)
    for b in range(B):
        for j in range(T):
            if not anc[i, j]:
                p = int(cl[b]) + j
                blk, off = table[b, p // bs], p % bs
                kp2[blk, :, off] = r.standard_normal(kp2[blk, :, off].shape)
                vp2[blk, :, off] = r.standard_normal(vp2[blk, :, off].shape)
    c = oracle.attention_dense(q, kp2, vp2, table, cl, tp, bs, "f32")
    assert np.max(np.abs(a[:, i] - c[:, i])) < 1e-12


@settings(**SETTINGS)
@given(tree_case(), st.integers(2, 6))
def test_greedy_path_invariants(case, V):
    parent, B, _, _, _, _, _, seed = case
    T = len(parent)
    rng = np.random.default_rng(seed)
    logits = rng.integers(-3, 4, size=(B, T, V)).astype(np.float32)   # many ties
    tok = rng.integers(0, V, size=(B, T)).astype(np.int32)
    tp = np.tile(parent, (B, 1))
    path, plen, bonus = oracle.accept(logits, "f32", None, tp, tok, np.zeros((B, T, 2), np.float32), 0.0)
    for b in range(B):
        L = int(plen[b])
        p = path[b, :L]
        assert p[0] == 0 and np.all(path[b, L:] == -1)
        for j in range(1, L):
            assert parent[p[j]] == p[j - 1]
            assert tok[b, p[j]] == int(np.argmax(logits[b, p[j - 1]]))
        last = int(p[-1])
        a = int(np.argmax(logits[b, last]))
        assert bonus[b] == a
        assert all(tok[b, c] != a for c in range(T) if parent[c] == last)


@settings(**SETTINGS)
@given(tree_case(), st.integers(0, 2 ** 31 - 1))
def test_commit_appends_the_path(case, seed2):
    parent, B, Hkv, G, D, bs, ctx, seed = case
    T = len(parent)
    q, kp, vp, table, cl, Kd, Vd = _cache(B, Hkv, G, D, bs, ctx, T, seed, shuffle_seed=seed)
    r = np.random.default_rng(seed2)
    path = np.full((B, T), -1, np.int32)
    plen = np.zeros(B, np.int32)
    for b in range(B):
        # a root path: walk down random children
        node, walk = 0, [0]
        while True:
            kids = [c for c in range(T) if parent[c] == node]
            if not kids or r.random() < 0.3:
                break
            node = int(r.choice(kids))
            walk.append(node)
        path[b, :len(walk)] = walk
        plen[b] = len(walk)
    K, V, c2 = oracle.commit(kp, vp, table, cl, path, plen, bs)
    assert np.array_equal(c2, cl + plen)
    touched = set()
    for b in range(B):
        c = int(cl[b])
        for t in range(c + int(plen[b])):
            blk, off = table[b, t // bs], t % bs
            src = t if t < c else c + int(path[b, t - c])
            assert np.array_equal(K[blk, :, off], Kd[b, :, src].astype(K.dtype))
            assert np.array_equal(V[blk, :, off], Vd[b, :, src].astype(V.dtype))
            if t >= c:
                touched.add((int(blk), off))
    for blk in range(kp.shape[0]):
        for off in range(bs):
            if (blk, off) not in touched:
                assert np.array_equal(K[blk, :, off], kp[blk, :, off])
