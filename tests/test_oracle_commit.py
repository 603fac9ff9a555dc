"""Pins for the commit oracle: identity paths, the in-place aliasing case,
untouched bytes, and the semantic check that attending over the committed
context equals attending over the old context plus the accepted path."""
import numpy as np

import oracle
from tests.helpers import paged_from_dense


def _cache(rng, B=2, n=40, Hkv=2, D=4, bs=4):
    Kd = rng.standard_normal((B, Hkv, n, D)).astype(np.float32)
    Vd = rng.standard_normal((B, Hkv, n, D)).astype(np.float32)
    return paged_from_dense(Kd, Vd, bs, rng, spare=2) + (Kd, Vd)


def _logical(kp, vp, table, b, p, bs):
    blk, off = table[b, p // bs], p % bs
    return kp[blk, :, off, :], vp[blk, :, off, :]


def test_identity_path_changes_nothing_but_lengths():
    rng = np.random.default_rng(0)
    kp, vp, table, Kd, Vd = _cache(rng)
    ctx = np.array([13, 21], np.int32)
    path = np.array([[0, 1, 2, -1], [0, -1, -1, -1]], np.int32)
    plen = np.array([3, 1], np.int32)
    K, V, c2 = oracle.commit(kp, vp, table, ctx, path, plen, 4)
    assert np.array_equal(K, kp) and np.array_equal(V, vp)
    assert list(c2) == [16, 22]


def test_aliasing_path_and_untouched_bytes():
    """path = [0, 2, 3]: slot ctx+1 takes slot ctx+2 while slot ctx+2 takes
    ctx+3 -- reads must see the old cache."""
    rng = np.random.default_rng(1)
    bs = 4
    kp, vp, table, Kd, Vd = _cache(rng, bs=bs)
    ctx = np.array([10, 7], np.int32)
    path = np.array([[0, 2, 3, -1, -1], [0, 1, 4, -1, -1]], np.int32)
    plen = np.array([3, 3], np.int32)
    K, V, c2 = oracle.commit(kp, vp, table, ctx, path, plen, bs)
    expect_src = {0: {10: 10, 11: 12, 12: 13}, 1: {7: 7, 8: 8, 9: 11}}
    for b in range(2):
        for p in range(40):
            kn, vn = _logical(K, V, table, b, p, bs)
            src = expect_src[b].get(p, p)
            assert np.array_equal(kn, Kd[b, :, src, :])
            assert np.array_equal(vn, Vd[b, :, src, :])
    # the spare blocks that no sequence maps are untouched
    used = set(table.ravel().tolist())
    for blk in range(kp.shape[0]):
        if blk not in used:
            assert np.array_equal(K[blk], kp[blk]) and np.array_equal(V[blk], vp[blk])
    assert list(c2) == [13, 10]


def test_committed_context_reproduces_path_attention():
    """After the commit, a single query over the new context equals the same
    query over the old context plus the accepted path as tree ancestors."""
    rng = np.random.default_rng(2)
    bs, D, T = 4, 8, 6
    Kd = rng.standard_normal((1, 1, 40, D)).astype(np.float32)
    Vd = rng.standard_normal((1, 1, 40, D)).astype(np.float32)
    kp, vp, table = paged_from_dense(Kd, Vd, bs)
    ctx = np.array([17], np.int32)
    parent = np.array([[-1, 0, 1, 1, 3, 0]], np.int32)
    path = np.array([[0, 1, 3, 4, -1, -1]], np.int32)
    plen = np.array([4], np.int32)
    qv = rng.standard_normal((1, T, 1, D)).astype(np.float32)
    before = oracle.attention_dense(qv, kp, vp, table, ctx, parent, bs, "f32")
    K, V, c2 = oracle.commit(kp, vp, table, ctx, path, plen, bs)
    # the deepest accepted node (4) is now the last committed token: a query
    # attending only to the committed context sees exactly its old key set
    q1 = qv[:, 4:5]
    after = oracle.attention_dense(q1, K, V, table, c2 - 1, np.array([[-1]], np.int32), bs, "f32")
    assert np.allclose(after[0, 0], before[0, 4], atol=1e-12)
