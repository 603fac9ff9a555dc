"""Pins for the block-selection oracle: integer-valued inputs where every
float32 operation is exact (so the score must equal the exact dot product),
error bounds against float64, a full sort by brute force on tiny inputs,
ties, partial blocks and planted high-norm blocks."""
import numpy as np
import pytest

import oracle
from synth.inputs import f32_to_bf16_bits
from tests.helpers import paged_from_dense


def _int_case(rng, B=2, Hkv=2, D=16, ctx=(20, 13), bs=4, T=3, Hq=4):
    """Small-integer keys and queries: every product and partial sum is an
    exact float32 integer, and block sums are multiples of the valid count."""
    n = max(ctx) + T
    Kd = rng.integers(-3, 4, size=(B, Hkv, n, D)).astype(np.float32)
    for b in range(B):
        for blk in range((ctx[b] + bs - 1) // bs):
            lo, hi = blk * bs, min(ctx[b], (blk + 1) * bs)
            # make each block's sum divisible by its valid count: mean is exact
            tot = Kd[b, :, lo:hi, :].sum(axis=1)
            Kd[b, :, hi - 1, :] -= np.mod(tot, hi - lo)
    Vd = np.zeros_like(Kd)
    q = rng.integers(-2, 3, size=(B, T, Hq, D)).astype(np.float32)
    kp, vp, table = paged_from_dense(Kd, Vd, bs, rng)
    return q, kp, table, np.array(ctx, np.int32), Kd


def test_exact_integer_scores_and_brute_force_sort():
    """Check (e): selection equals a brute-force full sort, with scores equal
    to the exact integer dot product of the query and the block-mean key."""
    rng = np.random.default_rng(0)
    bs = 4
    q, kp, table, ctx, Kd = _int_case(rng, bs=bs)
    means = oracle.block_means(kp, table, ctx, bs, "f32")
    for k in (1, 3, 5, 8, 9):
        sel = oracle.topk_blocks(q, kp, table, ctx, bs, k, "f32")
        for b in range(2):
            nb = (ctx[b] + bs - 1) // bs
            for i in range(3):
                for h in range(4):
                    g = h // 2
                    exact = []
                    for n in range(nb):
                        lo, hi = n * bs, min(ctx[b], (n + 1) * bs)
                        mean = [sum(int(Kd[b, g, t, d]) for t in range(lo, hi)) // (hi - lo)
                                for d in range(16)]
                        assert np.array_equal(means[b, n, g], np.array(mean, np.float32))
                        exact.append((-sum(int(q[b, i, h, d]) * mean[d] for d in range(16)), n))
                    best = sorted(n for _, n in sorted(exact)[:k])
                    want = best + [-1] * (k - len(best))
                    assert list(sel[b, i, h]) == want


def test_scores_within_float32_error_bound():
    rng = np.random.default_rng(1)
    D = 128
    qv = rng.standard_normal(D).astype(np.float32)
    m = rng.standard_normal((50, D)).astype(np.float32)
    s = oracle.block_scores(qv, m)
    exact = m.astype(np.float64) @ qv.astype(np.float64)
    bound = (np.abs(m.astype(np.float64)) @ np.abs(qv.astype(np.float64))) * 8 * 2.0 ** -24
    assert np.all(np.abs(s - exact) <= bound)


def test_block_mean_is_sequential_float32_sum():
    """The mean of a 64-token bf16 block equals the float64 mean within the
    float32 accumulation bound, and a partial block divides by its valid count."""
    rng = np.random.default_rng(2)
    bs, D = 64, 128
    Kf = rng.standard_normal((1, 1, 100, D)).astype(np.float32)
    Kb = f32_to_bf16_bits(Kf)
    kp, _, table = paged_from_dense(Kb, np.zeros_like(Kb), bs)
    means = oracle.block_means(kp, table, np.array([100], np.int32), bs, "bf16")
    Kx = (Kb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for n, (lo, hi) in enumerate([(0, 64), (64, 100)]):
        ref = Kx[0, 0, lo:hi].mean(axis=0)
        bound = np.abs(Kx[0, 0, lo:hi]).sum(axis=0) / (hi - lo) * (hi - lo + 1) * 2.0 ** -24
        assert np.all(np.abs(means[0, n, 0] - ref) <= bound)


def test_ties_go_to_lower_block_and_padding():
    """Duplicated blocks give exactly equal scores; the lower index wins."""
    rng = np.random.default_rng(3)
    bs, D = 2, 8
    base = rng.standard_normal((1, 1, 2, D)).astype(np.float32)
    Kd = np.concatenate([base] * 5, axis=2)           # 5 identical blocks
    kp, _, table = paged_from_dense(Kd, np.zeros_like(Kd), bs)
    q = rng.standard_normal((1, 1, 1, D)).astype(np.float32)
    sel = oracle.topk_blocks(q, kp, table, np.array([10], np.int32), bs, 3, "f32")
    assert list(sel[0, 0, 0]) == [0, 1, 2]
    sel = oracle.topk_blocks(q, kp, table, np.array([10], np.int32), bs, 7, "f32")
    assert list(sel[0, 0, 0]) == [0, 1, 2, 3, 4, -1, -1]
    sel = oracle.topk_blocks(q, kp, table, np.array([0], np.int32), bs, 2, "f32")
    assert list(sel[0, 0, 0]) == [-1, -1]


def test_planted_aligned_blocks_are_selected():
    rng = np.random.default_rng(4)
    bs, D, nblk = 16, 32, 20
    Kd = rng.standard_normal((1, 1, nblk * bs, D)).astype(np.float32)
    qv = rng.standard_normal(D).astype(np.float32)
    planted = [3, 11, 17]
    for n in planted:
        Kd[0, 0, n * bs:(n + 1) * bs] += 5.0 * qv / np.linalg.norm(qv)
    kp, _, table = paged_from_dense(Kd, np.zeros_like(Kd), bs, rng)
    sel = oracle.topk_blocks(qv[None, None, None], kp, table, np.array([nblk * bs], np.int32),
                             bs, 3, "f32")
    assert list(sel[0, 0, 0]) == planted


def test_block_sums_exact_integers():
    """Integer-valued keys: every float32 partial sum is exact, so each
    block's sum equals the exact integer sum of its valid rows (closed form)."""
    rng = np.random.default_rng(7)
    bs = 4
    q, kp, table, ctx, Kd = _int_case(rng, bs=bs)
    sums = oracle.block_sums(kp, table, ctx, bs, "f32")
    for b in range(2):
        for n in range((ctx[b] + bs - 1) // bs):
            lo, hi = n * bs, min(ctx[b], (n + 1) * bs)
            want = Kd[b, :, lo:hi, :].astype(np.float64).sum(axis=1)
            assert np.array_equal(sums[table[b, n]].astype(np.float64), want)
    # blocks no sequence holds as context stay NaN
    used = {int(table[b, n]) for b in range(2) for n in range((ctx[b] + bs - 1) // bs)}
    for blk in range(kp.shape[0]):
        if blk not in used:
            assert np.isnan(sums[blk]).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_means_from_sums_equal_means(dtype):
    """A mean formed from the kept sums is the very float32 value block_means
    forms from K (same sequential sum, same single division)."""
    rng = np.random.default_rng(11)
    B, Hkv, D, bs = 3, 2, 8, 8
    ctx = np.array([1, 17, 40], np.int32)
    n = 48
    Kd = rng.standard_normal((B, Hkv, n, D)).astype(np.float32)
    if dtype == "bf16":
        Kd = np.asarray(oracle.decode(f32_to_bf16_bits(Kd), "bf16"), np.float32)
    kp, vp, table = paged_from_dense(Kd if dtype == "f32" else Kd, np.zeros_like(Kd), bs, rng)
    if dtype == "bf16":
        kp = f32_to_bf16_bits(kp)
    sums = oracle.block_sums(kp, table, ctx, bs, dtype)
    a = oracle.means_from_sums(sums, table, ctx, bs)
    m = oracle.block_means(kp, table, ctx, bs, dtype)
    assert np.array_equal(a.view(np.uint32), m.view(np.uint32))


@pytest.mark.parametrize("ctx0,L", [(13, 5), (16, 8), (15, 1), (9, 0), (0, 3)])
def test_append_block_sums_equals_rebuild(ctx0, L):
    """Extending the sums by the positions a commit appended gives the sums
    rebuilt from scratch at the new length, bit for bit: across a block
    boundary, starting a new block, a single position, nothing, and an empty
    context."""
    rng = np.random.default_rng(ctx0 * 31 + L)
    B, Hkv, D, bs = 2, 2, 8, 8
    n = 40
    Kd = rng.standard_normal((B, Hkv, n, D)).astype(np.float32)
    kp, vp, table = paged_from_dense(Kd, np.zeros_like(Kd), bs, rng)
    ctx = np.array([ctx0, ctx0 + 3], np.int32)
    sums = oracle.block_sums(kp, table, ctx, bs, "f32")
    plen = np.array([L, L], np.int32)
    ctx_new = ctx + plen
    got = oracle.append_block_sums(sums, kp, table, ctx_new, plen, bs, "f32")
    want = oracle.block_sums(kp, table, ctx_new, bs, "f32")
    live = ~np.isnan(want)
    assert np.array_equal(got[live].view(np.uint32), want[live].view(np.uint32))


def test_shared_selection_exact_integers_brute_force():
    """Shared selection: with exact integer arithmetic the score is the sum
    of the group's per-row dot products; the selection equals a full sort of
    that exact sum, and every row of a group holds the same list."""
    rng = np.random.default_rng(11)
    bs = 4
    q, kp, table, ctx, Kd = _int_case(rng, bs=bs)
    G = 2
    for k in (1, 2, 4, 5, 9):
        sel = oracle.topk_blocks_shared(q, kp, table, ctx, bs, k, "f32")
        for b in range(2):
            nb = (ctx[b] + bs - 1) // bs
            for g in range(2):
                exact = []
                for n in range(nb):
                    lo, hi = n * bs, min(ctx[b], (n + 1) * bs)
                    mean = [sum(int(Kd[b, g, t, d]) for t in range(lo, hi)) // (hi - lo) for d in range(16)]
                    tot = sum(int(q[b, i, g * G + j, d]) * mean[d]
                              for i in range(3) for j in range(G) for d in range(16))
                    exact.append((-tot, n))
                best = sorted(n for _, n in sorted(exact)[:k])
                want = best + [-1] * (k - len(best))
                for i in range(3):
                    for j in range(G):
                        assert list(sel[b, i, g * G + j]) == want


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shared_selection_reduces_to_per_row(dtype):
    """One query row per KV group (T = 1, Hq = Hkv): the shared selection is
    the per-row selection.  With every other row of a group zero, it is the
    one nonzero row's selection (adding +0 leaves a float32 sum unchanged)."""
    rng = np.random.default_rng(12)
    B, Hkv, D, bs = 2, 3, 32, 8
    ctx = (70, 45)
    Kd = rng.standard_normal((B, Hkv, max(ctx) + 4, D)).astype(np.float32)
    kp, _, table = paged_from_dense(Kd, np.zeros_like(Kd), bs, rng)
    if dtype == "bf16":
        kp = f32_to_bf16_bits(kp)
    ctx = np.array(ctx, np.int32)
    q1 = rng.standard_normal((B, 1, Hkv, D)).astype(np.float32)
    if dtype == "bf16":
        q1 = f32_to_bf16_bits(q1)
    for k in (1, 3, 6):
        assert np.array_equal(oracle.topk_blocks_shared(q1, kp, table, ctx, bs, k, dtype),
                              oracle.topk_blocks(q1, kp, table, ctx, bs, k, dtype))
    # T = 4, G = 2: only node 2, head 1 of each group is nonzero
    q = np.zeros((B, 4, 2 * Hkv, D), np.float32)
    q[:, 2, 1::2] = rng.standard_normal((B, Hkv, D))
    if dtype == "bf16":
        q = f32_to_bf16_bits(q)
    per_row = oracle.topk_blocks(q, kp, table, ctx, bs, 5, dtype)
    shared = oracle.topk_blocks_shared(q, kp, table, ctx, bs, 5, dtype)
    for g in range(Hkv):
        for i in range(4):
            for j in range(2):
                assert np.array_equal(shared[:, i, 2 * g + j], per_row[:, 2, 2 * g + 1])
