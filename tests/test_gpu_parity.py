"""GPU parity: every C-ABI call against the CPU oracle on the same seeded
inputs -- small variants of the five workloads in full, the full-size
workloads on sampled outputs, and edge cases."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_inputs, small_variant
from synth.configs import CONFIG_ORDER
from tests.devutil import check_attention, compare_accept, dev_tensor, host_f64, to_device

pytestmark = pytest.mark.gpu

tva = pytest.importorskip("tree_verification_amd")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _tau(c):
    return 0.0 if c.mode == "greedy" else c.temperature


def _run_attn(x, d, sel=None):
    out = tva.tree_verify_attn(d["q"], d["k"], d["v"], d["table"], d["ctx"], d["parent"],
                               sel_blocks=None if sel is None else dev_tensor(sel))
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    return host_f64(out)


SMALL = CONFIG_ORDER


@pytest.mark.parametrize("name", SMALL)
def test_attention_small_full_compare(name):
    c = small_variant(name)
    _say("attention small %s" % name)
    x = make_inputs(c)
    d = to_device(x)
    gpu = _run_attn(x, d)
    ref = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens,
                                 x.tree_parent, c.bs, c.dtype)
    check_attention(gpu, ref, c.dtype, name)


# Shapes whose (sequence, KV head, 256-row query tile) count fills the chip
# without a context split: the bf16 path then runs its 256-row workgroups over
# 32-key tiles (ragged contexts, a ragged tree tail, a deep best-first tree
# whose far tree tiles are skipped).
WIDE_TILE = {
    "tree64": ("llama3_8b_tree64", dict(B=32, ctx_lo=61, ctx_hi=190)),
    "tree200": ("llama3_8b_tree64", dict(B=32, T=200, ctx_lo=40, ctx_hi=97)),
    "bestfirst1024": ("specexec_70b_tree2048", dict(T=1024, ctx_lo=77, ctx_hi=77, V=700)),
}


@pytest.mark.parametrize("case", sorted(WIDE_TILE))
def test_attention_wide_query_tile(case):
    name, over = WIDE_TILE[case]
    c = small_variant(name, **over)
    M = c.T * (c.Hq // c.Hkv)
    assert c.dtype == "bf16" and c.D == 128 and M > 128 and c.B * c.Hkv * ((M + 255) // 256) >= 256
    _say("attention wide query tile %s" % case)
    x = make_inputs(c)
    d = to_device(x)
    gpu = _run_attn(x, d)
    ref = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens,
                                 x.tree_parent, c.bs, c.dtype)
    check_attention(gpu, ref, c.dtype, case)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", ["T1", "ctx0", "shared_tree", "forest", "ragged_tail", "gqa1",
                                  "d64", "chain_deep", "wide_T"])
def test_attention_edge_cases(case, dtype):
    over = {
        "T1": dict(T=1, tree="chain"),
        "ctx0": dict(ctx_lo=0, ctx_hi=0),
        "shared_tree": dict(),
        "forest": dict(),
        "ragged_tail": dict(ctx_lo=63, ctx_hi=65, bs=8),
        "gqa1": dict(Hq=8, Hkv=8),
        "d64": dict(D=64),
        "chain_deep": dict(tree="chain", T=70),
        "wide_T": dict(T=200, max_parent_depth=3, max_children=40, ctx_lo=100, ctx_hi=150),
    }[case]
    c = small_variant("llama3_8b_tree64", **{**dict(B=2, ctx_lo=37, ctx_hi=77, T=20, dtype=dtype),
                                             **over})
    _say("attention edge %s %s" % (case, dtype))
    x = make_inputs(c)
    if case == "shared_tree":
        x.tree_parent = x.tree_parent[:1].copy()
    if case == "forest":
        x.tree_parent[:, 5] = -1
        x.tree_parent[:, 11] = -1
    d = to_device(x)
    gpu = _run_attn(x, d)
    ref = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens,
                                 x.tree_parent, c.bs, c.dtype)
    check_attention(gpu, ref, c.dtype, case)


def _pad_table(x, width):
    """Widens the block table to `width` columns of -1: the launch plan then
    sees a larger cache capacity (more key tiles, more context splits)
    without any longer context."""
    mb = x.block_table.shape[1]
    x.block_table = np.pad(x.block_table, ((0, 0), (0, width - mb)), constant_values=-1)


def test_attention_split_shapes_share_a_workspace():
    """Split launches of different shapes in a row, on the binding's one
    attention workspace (partials of one shape left where the next one's
    lie)."""
    cases = [dict(B=3), dict(B=5, ctx_lo=300, ctx_hi=700), dict(B=3)]
    for over in cases:
        c = small_variant("longctx_paged_tree16", **over)
        _say("attention split shapes B=%d" % c.B)
        x = make_inputs(c)
        d = to_device(x)
        gpu = _run_attn(x, d)
        ref = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens,
                                     x.tree_parent, c.bs, c.dtype)
        check_attention(gpu, ref, c.dtype, "split shapes B=%d" % c.B)


def test_attention_many_units_split():
    """A large split launch: 520 sequences x 8 KV heads, their contexts short
    but their block table 2100 blocks wide, so that the plan splits each
    (sequence, KV head) in two by its block-id limit (8320 workgroups)."""
    c = small_variant("llama3_8b_tree64", B=520, T=4, ctx_lo=20, ctx_hi=60, V=257)
    _say("attention many units: generating")
    x = make_inputs(c)
    _pad_table(x, 2100)
    d = to_device(x)
    _say("attention many units: running")
    gpu = _run_attn(x, d)
    ref = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens,
                                 x.tree_parent, c.bs, c.dtype)
    check_attention(gpu, ref, c.dtype, "many units")


def _sample_rows(c, n, seed):
    r = np.random.default_rng(seed)
    rows = {(int(r.integers(c.B)), int(r.integers(c.T)), int(r.integers(c.Hq))) for _ in range(n)}
    rows |= {(0, 0, 0), (c.B - 1, c.T - 1, c.Hq - 1)}
    return sorted(rows)


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_attention_full_size_sampled(name):
    c = CONFIGS[name]
    _say("attention full %s: generating" % name)
    x = make_inputs(c)
    d = to_device(x)
    _say("attention full %s: running" % name)
    gpu = _run_attn(x, d)
    rows = _sample_rows(c, 24, 1)
    ref = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens,
                                 x.tree_parent, c.bs, c.dtype, rows=rows)
    got = np.stack([gpu[b, i, h] for b, i, h in rows])
    check_attention(got, ref, c.dtype, name)


def _accept_both(c, x, d):
    tau = _tau(c)
    draft = d["draft"] if c.mode == "mss" else None
    p, l, b = tva.accept(d["logits"], draft, d["parent"], d["token"], d["unif"], tau)
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    gpu = (p.cpu().numpy(), l.cpu().numpy(), b.cpu().numpy())
    ref = oracle.accept(x.target_logits, c.logit_dtype, x.draft_probs if c.mode == "mss" else None,
                        x.tree_parent, x.tree_token, x.uniforms, tau, trace=True)
    return gpu, ref


@pytest.mark.parametrize("name", CONFIG_ORDER)
@pytest.mark.parametrize("size", ["small", "full"])
def test_accept(name, size):
    c = small_variant(name) if size == "small" else CONFIGS[name]
    _say("accept %s %s" % (size, name))
    x = make_inputs(c)
    d = to_device(x)
    gpu, ref = _accept_both(c, x, d)
    compare_accept(gpu, ref[:3], ref[3])
    if name == "specexec_70b_tree2048":
        c2 = dataclasses.replace(c, mode="greedy", temperature=0.0)
        gpu, ref = _accept_both(c2, x, d)
        compare_accept(gpu, ref[:3], ref[3])


@pytest.mark.parametrize("L", range(0, 6))
def test_accept_greedy_planted_prefix(L):
    T, V = 6, 50
    rng = np.random.default_rng(L)
    logits = rng.standard_normal((1, T, V)).astype(np.float32)
    tokens = np.zeros((1, T), np.int32)
    for j in range(T):
        a = (3 * j + 5) % V
        logits[0, j, a] = 10.0
        if j + 1 < T:
            tokens[0, j + 1] = a if j < L else (a + 1) % V
    parent = np.arange(-1, T - 1, dtype=np.int32)[None]
    p, l, b = tva.accept(dev_tensor(logits), None, dev_tensor(parent), dev_tensor(tokens), None, 0.0)
    assert l.item() == L + 1 and b.item() == (3 * L + 5) % V
    assert p.cpu().numpy()[0, :L + 1].tolist() == list(range(L + 1))


def test_accept_ties_and_duplicates():
    V = 10
    logits = np.zeros((1, 5, V), np.float32)
    logits[0, 0, [4, 2, 8]] = 3.0
    logits[0, 2, 6] = 1.0
    parent = np.array([[-1, 0, 0, 0, 2]], np.int32)
    tokens = np.array([[0, 4, 2, 2, 6]], np.int32)
    p, l, b = tva.accept(dev_tensor(logits), None, dev_tensor(parent), dev_tensor(tokens), None, 0.0)
    assert p.cpu().numpy()[0, :l.item()].tolist() == [0, 2, 4] and b.item() == 0


def test_accept_rejects_bad_tree():
    logits = np.zeros((2, 4, 16), np.float32)
    parent = np.array([[-1, 0, 2, 1], [-1, 0, 0, 1]], np.int32)     # node 2 of seq 0 points forward
    tokens = np.array([[0, 1, 2, 3], [0, 1, 2, 99]], np.int32)      # token 99 out of range
    p, l, b = tva.accept(dev_tensor(logits), None, dev_tensor(parent), dev_tensor(tokens), None, 0.0)
    torch.cuda.synchronize()
    bits = tva.device_status()
    assert bits & 0x1 and bits & 0x8
    assert l.cpu().tolist() == [0, 0]


def test_rejection_sampling_distribution_1e6():
    """Check (d) on the GPU: vocabulary 8, 10^6 independent trials, four i.i.d.
    siblings; first emitted token vs softmax(l / tau), chi-square p > 0.01."""
    from scipy import stats
    from scipy.special import softmax
    n, V, nc, tau = 1_000_000, 8, 4, 0.8
    rng = np.random.default_rng(123)
    pl = np.array([1.2, -0.3, 0.4, 2.0, -1.0, 0.0, 0.9, -2.2], np.float32)
    q = np.array([0.05, 0.30, 0.05, 0.10, 0.25, 0.05, 0.15, 0.05])
    T = 1 + nc
    parent = np.tile(np.array([-1] + [0] * nc, np.int32), (n, 1))
    tokens = np.zeros((n, T), np.int32)
    tokens[:, 1:] = rng.choice(V, size=(n, nc), p=q)
    logits = np.ascontiguousarray(np.broadcast_to(pl, (n, T, V)))
    qd = np.ascontiguousarray(np.broadcast_to(q.astype(np.float32), (n, T, V)))
    unif = (rng.integers(0, 1 << 24, size=(n, T, 2)) * 2.0 ** -24).astype(np.float32)
    p, l, b = tva.accept(dev_tensor(logits), dev_tensor(qd), dev_tensor(parent), dev_tensor(tokens),
                         dev_tensor(unif), tau)
    p, l, b = p.cpu().numpy(), l.cpu().numpy(), b.cpu().numpy()
    first = np.where(l > 1, tokens[np.arange(n), np.maximum(p[:, 1], 0)], b)
    obs = np.bincount(first, minlength=V)
    exp = softmax(pl.astype(np.float64) / tau) * n
    assert stats.chisquare(obs, exp).pvalue > 0.01
    # the same uniforms through the oracle on a slice agree exactly
    sl = slice(0, 2000)
    ref = oracle.accept(logits[sl], "f32", qd[sl], parent[sl], tokens[sl], unif[sl], tau)
    assert np.array_equal(ref[1], l[sl]) and np.array_equal(ref[2], b[sl])


def _commit_case(c):
    x = make_inputs(c)
    d = to_device(x)
    tau = _tau(c)
    path, plen, _ = oracle.accept(x.target_logits, c.logit_dtype,
                                  x.draft_probs if c.mode == "mss" else None,
                                  x.tree_parent, x.tree_token, x.uniforms, tau)
    return x, d, path, plen


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_commit_bit_exact(name):
    c = small_variant(name)
    _say("commit %s" % name)
    x, d, path, plen = _commit_case(c)
    K, V, ctx2 = oracle.commit(x.k_pages, x.v_pages, x.block_table, x.ctx_lens, path, plen, c.bs)
    tva.kv_commit(d["k"], d["v"], d["table"], d["ctx"], dev_tensor(path), dev_tensor(plen))
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    kd = d["k"].view(torch.int16).cpu().numpy().view(x.k_pages.dtype) if c.dtype == "bf16" \
        else d["k"].cpu().numpy()
    vd = d["v"].view(torch.int16).cpu().numpy().view(x.v_pages.dtype) if c.dtype == "bf16" \
        else d["v"].cpu().numpy()
    assert np.array_equal(kd.view(np.uint8), K.view(np.uint8))
    assert np.array_equal(vd.view(np.uint8), V.view(np.uint8))
    assert np.array_equal(d["ctx"].cpu().numpy(), ctx2)


def test_commit_aliasing_path():
    c = small_variant("llama3_8b_tree64", B=2, T=8, tree="chain", ctx_lo=21, ctx_hi=30)
    x = make_inputs(c)
    d = to_device(x)
    path = np.array([[0, 2, 3, 5, 7, -1, -1, -1], [0, 1, 2, 3, 4, 5, 6, 7]], np.int32)
    plen = np.array([5, 8], np.int32)
    K, V, ctx2 = oracle.commit(x.k_pages, x.v_pages, x.block_table, x.ctx_lens, path, plen, c.bs)
    tva.kv_commit(d["k"], d["v"], d["table"], d["ctx"], dev_tensor(path), dev_tensor(plen))
    torch.cuda.synchronize()
    assert np.array_equal(d["k"].view(torch.int16).cpu().numpy().view(np.uint16), K)
    assert np.array_equal(d["v"].view(torch.int16).cpu().numpy().view(np.uint16), V)
    assert np.array_equal(d["ctx"].cpu().numpy(), ctx2)


def _topk_case(c):
    x = make_inputs(c)
    d = to_device(x)
    sel = tva.topk_blocks(d["q"], d["k"], d["table"], d["ctx"], c.topk)
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    ref = oracle.topk_blocks(x.q, x.k_pages, x.block_table, x.ctx_lens, c.bs, c.topk, c.dtype)
    return x, d, sel.cpu().numpy(), ref


@pytest.mark.parametrize("size", ["small", "full"])
def test_topk_bit_exact(size):
    name = "sparse_topk32_ctx64k"
    c = small_variant(name) if size == "small" else CONFIGS[name]
    _say("topk %s" % size)
    x, d, sel, ref = _topk_case(c)
    assert np.array_equal(sel, ref)


@pytest.mark.parametrize("k", [1, 3, 9, 40])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_topk_edge_k(k, dtype):
    c = small_variant("sparse_topk32_ctx64k", topk=k, dtype=dtype, ctx_lo=0, ctx_hi=700, B=3)
    x, d, sel, ref = _topk_case(c)
    assert np.array_equal(sel, ref)


@pytest.mark.parametrize("size", ["small", "full"])
def test_sparse_attention(size):
    name = "sparse_topk32_ctx64k"
    c = small_variant(name) if size == "small" else CONFIGS[name]
    _say("sparse attention %s" % size)
    x = make_inputs(c)
    d = to_device(x)
    ref_sel = oracle.topk_blocks(x.q, x.k_pages, x.block_table, x.ctx_lens, c.bs, c.topk, c.dtype)
    gpu = _run_attn(x, d, sel=ref_sel)
    if size == "small":
        ref = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens,
                                     x.tree_parent, c.bs, c.dtype, sel_blocks=ref_sel)
        check_attention(gpu, ref, c.dtype, "sparse small")
    else:
        rows = _sample_rows(c, 24, 2)
        ref = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens,
                                     x.tree_parent, c.bs, c.dtype, sel_blocks=ref_sel, rows=rows)
        check_attention(np.stack([gpu[b, i, h] for b, i, h in rows]), ref, c.dtype, "sparse full")


@pytest.mark.parametrize("k", [100, 200])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sparse_attention_wide_selection(k, dtype):
    """Selections of more than 64 blocks per query row (the sparse-verification
    page's k trade-off reaches past 64): the library's top-k of a context of
    1500-2500 tokens in blocks of 8 (188-313 blocks) equals the oracle's, and
    the attention over it matches the oracle's attention over the same lists."""
    c = small_variant("sparse_topk32_ctx64k", topk=k, dtype=dtype, bs=8, ctx_lo=1500, ctx_hi=2500, B=2)
    _say("sparse wide k=%d %s" % (k, dtype))
    x, d, sel, ref_sel = _topk_case(c)
    assert np.array_equal(sel, ref_sel)
    gpu = _run_attn(x, d, sel=ref_sel)
    ref = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens,
                                 x.tree_parent, c.bs, c.dtype, sel_blocks=ref_sel)
    check_attention(gpu, ref, c.dtype, "sparse wide")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sparse_attention_fp32_and_partial_selection(dtype):
    c = small_variant("sparse_topk32_ctx64k", dtype=dtype, B=2, ctx_lo=300, ctx_hi=500, bs=16)
    x = make_inputs(c)
    d = to_device(x)
    rng = np.random.default_rng(9)
    ks = 5
    sel = np.full((c.B, c.T, c.Hq, ks), -1, np.int32)
    for b in range(c.B):
        nb = (int(x.ctx_lens[b]) + c.bs - 1) // c.bs
        for i in range(c.T):
            for h in range(c.Hq):
                m = int(rng.integers(0, ks + 1))
                sel[b, i, h, :m] = np.sort(rng.choice(nb, size=m, replace=False))
    gpu = _run_attn(x, d, sel=sel)
    ref = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens,
                                 x.tree_parent, c.bs, c.dtype, sel_blocks=sel)
    check_attention(gpu, ref, c.dtype, "sparse random sel")


def test_bad_block_id_sets_status():
    c = small_variant("llama3_8b_tree64", B=2, T=8, ctx_lo=40, ctx_hi=40)
    x = make_inputs(c)
    x.block_table[1, 1] = x.k_pages.shape[0] + 5
    d = to_device(x)
    tva.tree_verify_attn(d["q"], d["k"], d["v"], d["table"], d["ctx"], d["parent"])
    torch.cuda.synchronize()
    assert tva.device_status() & 0x2


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bad_parent_sets_status(dtype):
    c = small_variant("llama3_8b_tree64", B=2, T=8, ctx_lo=40, ctx_hi=40, dtype=dtype)
    x = make_inputs(c)
    x.tree_parent[1, 5] = 6                       # points forward
    d = to_device(x)
    _say("attention bad parent %s" % dtype)
    tva.tree_verify_attn(d["q"], d["k"], d["v"], d["table"], d["ctx"], d["parent"])
    torch.cuda.synchronize()
    assert tva.device_status() & 0x1
    x.tree_parent[1, 5] = x.tree_parent[1, 4]     # valid again: no bit
    d = to_device(x)
    tva.tree_verify_attn(d["q"], d["k"], d["v"], d["table"], d["ctx"], d["parent"])
    torch.cuda.synchronize()
    assert tva.device_status() == 0
