"""Pins for the attention oracle: it is checked against torch's
scaled_dot_product_attention (an independent implementation), closed forms,
brute force over every tree of up to five nodes, and invariances."""
import numpy as np
import pytest
import torch

import oracle
from synth import make_inputs, small_variant
from tests.helpers import all_trees, paged_from_dense, path_by_walk


def sdpa(qv, K, V, scale, mask=None):
    """torch reference, float64, one query row."""
    q = torch.tensor(qv, dtype=torch.float64)[None, None, None, :]
    k = torch.tensor(K, dtype=torch.float64)[None, None]
    v = torch.tensor(V, dtype=torch.float64)[None, None]
    m = None if mask is None else torch.tensor(mask)[None, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)
    return o[0, 0, 0].numpy()


def _rand_case(rng, B=2, T=5, Hq=4, Hkv=2, D=16, ctx=(7, 13), bs=4, parent=None, shuffle=True):
    n = max(ctx) + T
    Kd = rng.standard_normal((B, Hkv, n, D))
    Vd = rng.standard_normal((B, Hkv, n, D))
    q = rng.standard_normal((B, T, Hq, D))
    kp, vp, table = paged_from_dense(Kd, Vd, bs, rng if shuffle else None, spare=2)
    ctx_lens = np.array(ctx[:B], dtype=np.int32)
    if parent is None:
        parent = np.array([-1] + [int(rng.integers(i)) for i in range(1, T)], dtype=np.int32)
    tp = np.tile(parent, (B, 1))
    return q, kp, vp, table, ctx_lens, tp, Kd, Vd


def test_dense_equals_per_path_formulation():
    """Check (a): each node's output equals ordinary causal attention along its
    own root path.  Both formulations, on the synthetic small workloads."""
    for name in ["llama3_8b_tree64", "longctx_paged_tree16", "specexec_70b_tree2048"]:
        c = small_variant(name, B=1, Hq=16, Hkv=8, ctx_lo=40, ctx_hi=57, T=min(small_variant(name).T, 24))
        x = make_inputs(c)
        a = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens,
                                   x.tree_parent, c.bs, c.dtype)
        b = oracle.attention_by_path(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens,
                                     x.tree_parent, c.bs, c.dtype)
        assert np.max(np.abs(a - b)) < 1e-12


def test_every_tree_up_to_five_nodes_against_sdpa():
    """Brute force: all 34 trees with <= 5 nodes; every node against torch SDPA
    run on [context, root path] with no mask."""
    rng = np.random.default_rng(1)
    for T in range(1, 6):
        for parent in all_trees(T):
            q, kp, vp, table, ctx_lens, tp, Kd, Vd = _rand_case(rng, B=1, T=T, Hq=2, Hkv=1, D=8,
                                                                ctx=(5,), bs=3, parent=parent)
            out = oracle.attention_dense(q, kp, vp, table, ctx_lens, tp, 3, "f32")
            ctx = int(ctx_lens[0])
            for i in range(T):
                keys = list(range(ctx)) + [ctx + j for j in path_by_walk(parent, i)]
                for h in range(2):
                    ref = sdpa(q[0, i, h], Kd[0, 0, keys], Vd[0, 0, keys], 8 ** -0.5)
                    # the oracle stores float32-typed inputs; compare at float32 input precision
                    assert np.allclose(out[0, i, h], ref, atol=1e-6), (parent, i, h)


def test_chain_is_causal_multitoken_attention():
    """Check (b): a chain-shaped tree is standard causal multi-token attention
    with a KV prefix.  torch SDPA with an explicit causal mask over all heads."""
    rng = np.random.default_rng(2)
    T, ctx, Hq, Hkv, D = 6, 11, 4, 2, 16
    parent = np.arange(-1, T - 1, dtype=np.int32)
    q, kp, vp, table, ctx_lens, tp, Kd, Vd = _rand_case(rng, B=1, T=T, Hq=Hq, Hkv=Hkv, D=D,
                                                        ctx=(ctx,), bs=4, parent=parent)
    q = q.astype(np.float32)
    kp = kp.astype(np.float32)
    vp = vp.astype(np.float32)
    Kd = Kd.astype(np.float32).astype(np.float64)
    Vd = Vd.astype(np.float32).astype(np.float64)
    out = oracle.attention_dense(q, kp, vp, table, ctx_lens, tp, 4, "f32")
    G = Hq // Hkv
    n = ctx + T
    mask = np.zeros((T, n), dtype=bool)
    for i in range(T):
        mask[i, :ctx + i + 1] = True
    Q = torch.tensor(q[0].astype(np.float64)).permute(1, 0, 2)              # [Hq, T, D]
    K = torch.tensor(Kd[0]).repeat_interleave(G, dim=0)                     # [Hq, n, D]
    V = torch.tensor(Vd[0]).repeat_interleave(G, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q[None], K[None], V[None], attn_mask=torch.tensor(mask)[None, None])[0]
    assert np.max(np.abs(out[0] - ref.permute(1, 0, 2).numpy())) < 1e-12


def test_identical_keys_give_mean_of_visible_values():
    """Closed form: if every key is the same vector the softmax is uniform, so
    the output is the plain mean of V over exactly the visible set."""
    rng = np.random.default_rng(3)
    T, ctx, D = 7, 9, 8
    parent = np.array([-1, 0, 0, 1, 3, 2, 4], dtype=np.int32)
    Kd = np.tile(rng.standard_normal(D), (1, 1, ctx + T, 1))
    Vd = rng.standard_normal((1, 1, ctx + T, D))
    kp, vp, table = paged_from_dense(Kd, Vd, 5, rng)
    q = rng.standard_normal((1, T, 1, D))
    out = oracle.attention_dense(q, kp, vp, table, np.array([ctx], np.int32), parent[None], 5, "f32")
    Vf = Vd.astype(np.float32).astype(np.float64)
    for i in range(T):
        vis = list(range(ctx)) + [ctx + j for j in path_by_walk(parent, i)]
        assert np.allclose(out[0, i, 0], Vf[0, 0, vis].mean(axis=0), atol=1e-6)


def test_dominant_key_selects_its_value():
    """Closed form: with one visible key far above the rest, the output is that
    key's value; keys that must stay hidden (siblings, descendants) carry even
    larger scores, so any mask leak changes the answer."""
    T, ctx, D = 6, 4, 4
    parent = np.array([-1, 0, 0, 1, 1, 3], dtype=np.int32)
    e0 = np.zeros(D)
    e0[0] = 1.0
    Kd = np.zeros((1, 1, ctx + T, D))
    # tree node j's key grows with j, so the deepest visible ancestor wins
    for j in range(T):
        Kd[0, 0, ctx + j] = e0 * (10.0 * (j + 1))
    Vd = np.zeros((1, 1, ctx + T, D))
    for p in range(ctx + T):
        Vd[0, 0, p, 1] = p
    kp, vp, table = paged_from_dense(Kd, Vd, 3)
    q = np.tile(e0 * 4.0, (1, T, 1, 1))
    out = oracle.attention_dense(q, kp, vp, table, np.array([ctx], np.int32), parent[None], 3, "f32",
                                 scale=1.0)
    for i in range(T):
        deepest = max(path_by_walk(parent, i))
        assert abs(out[0, i, 0, 1] - (ctx + deepest)) < 1e-6


def test_single_node_is_decode_and_empty_context_is_tree_only():
    rng = np.random.default_rng(4)
    # T = 1: one query over ctx + 1 keys
    q, kp, vp, table, ctx_lens, tp, Kd, Vd = _rand_case(rng, B=1, T=1, Hq=1, Hkv=1, D=8, ctx=(10,),
                                                        bs=4, parent=np.array([-1], np.int32))
    out = oracle.attention_dense(q, kp, vp, table, ctx_lens, tp, 4, "f32")
    ref = sdpa(q[0, 0, 0].astype(np.float32), Kd[0, 0, :11].astype(np.float32),
               Vd[0, 0, :11].astype(np.float32), 8 ** -0.5)
    assert np.allclose(out[0, 0, 0], ref, atol=1e-9)
    # ctx = 0: ancestors only
    parent = np.array([-1, 0, 1, 0], dtype=np.int32)
    q, kp, vp, table, ctx_lens, tp, Kd, Vd = _rand_case(rng, B=1, T=4, Hq=1, Hkv=1, D=8, ctx=(0,),
                                                        bs=4, parent=parent)
    out = oracle.attention_dense(q, kp, vp, table, ctx_lens, tp, 4, "f32")
    for i in range(4):
        keys = path_by_walk(parent, i)
        ref = sdpa(q[0, i, 0].astype(np.float32), Kd[0, 0, keys].astype(np.float32),
                   Vd[0, 0, keys].astype(np.float32), 8 ** -0.5)
        assert np.allclose(out[0, i, 0], ref, atol=1e-9)


def test_page_placement_does_not_matter():
    """Shuffling physical blocks (with the table updated) leaves outputs unchanged."""
    rng = np.random.default_rng(5)
    B, T, Hq, Hkv, D, bs = 2, 5, 4, 2, 8, 4
    Kd = rng.standard_normal((B, Hkv, 30, D))
    Vd = rng.standard_normal((B, Hkv, 30, D))
    q = rng.standard_normal((B, T, Hq, D))
    parent = np.tile(np.array([-1, 0, 0, 2, 1], np.int32), (B, 1))
    ctx = np.array([25, 17], np.int32)
    a = oracle.attention_dense(q, *paged_from_dense(Kd, Vd, bs), ctx, parent, bs, "f32")
    b = oracle.attention_dense(q, *paged_from_dense(Kd, Vd, bs, rng, spare=3), ctx, parent, bs, "f32")
    assert np.max(np.abs(a - b)) == 0.0


def test_sparse_selection_restricts_context_only():
    rng = np.random.default_rng(6)
    T, ctx, D, bs = 4, 19, 8, 4
    parent = np.array([-1, 0, 1, 1], np.int32)
    q, kp, vp, table, ctx_lens, tp, Kd, Vd = _rand_case(rng, B=1, T=T, Hq=2, Hkv=1, D=D, ctx=(ctx,),
                                                        bs=bs, parent=parent)
    nblk = (ctx + bs - 1) // bs
    full = np.tile(np.arange(nblk, dtype=np.int32), (1, T, 2, 1))
    dense = oracle.attention_dense(q, kp, vp, table, ctx_lens, tp, bs, "f32")
    sp = oracle.attention_dense(q, kp, vp, table, ctx_lens, tp, bs, "f32", sel_blocks=full)
    assert np.max(np.abs(dense - sp)) < 1e-15
    sel = np.full((1, T, 2, 3), -1, np.int32)
    sel[0, :, 0, :2] = [1, 4]          # block 4 is the partial last context block
    out = oracle.attention_dense(q, kp, vp, table, ctx_lens, tp, bs, "f32", sel_blocks=sel)
    alt = oracle.attention_by_path(q, kp, vp, table, ctx_lens, tp, bs, "f32", sel_blocks=sel)
    assert np.max(np.abs(out - alt)) < 1e-12
    for i in range(T):
        path = [ctx + j for j in path_by_walk(parent, i)]
        keys0 = [p for p in range(ctx) if p // bs in (1, 4)] + path
        ref0 = sdpa(q[0, i, 0].astype(np.float32), Kd[0, 0, keys0].astype(np.float32),
                    Vd[0, 0, keys0].astype(np.float32), D ** -0.5)
        ref1 = sdpa(q[0, i, 1].astype(np.float32), Kd[0, 0, path].astype(np.float32),
                    Vd[0, 0, path].astype(np.float32), D ** -0.5)
        assert np.allclose(out[0, i, 0], ref0, atol=1e-9)
        assert np.allclose(out[0, i, 1], ref1, atol=1e-9)


def test_rows_subset_matches_full():
    c = small_variant("llama3_8b_tree64", B=2, ctx_lo=33, ctx_hi=40, T=12)
    x = make_inputs(c)
    full = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens,
                                  x.tree_parent, c.bs, c.dtype)
    rows = [(0, 0, 0), (1, 11, 31), (1, 5, 7), (0, 3, 12)]
    sub = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens,
                                 x.tree_parent, c.bs, c.dtype, rows=rows)
    for r, (b, i, h) in enumerate(rows):
        assert np.array_equal(sub[r], full[b, i, h])
