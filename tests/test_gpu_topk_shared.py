"""sd_topk_blocks_shared on the GPU against the oracle: one selection per
(sequence, KV group), bit for bit, from K and from kept block sums; and
sparse attention over the shared selection against the oracle's attention."""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_inputs, small_variant
from tests.devutil import check_attention, host_f64, to_device

tva = pytest.importorskip("tree_verification_amd")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = {
    "sparse_small": lambda: small_variant("sparse_topk32_ctx64k"),
    "sparse_small_f32": lambda: small_variant("sparse_topk32_ctx64k", dtype="f32"),
    "longctx_shuffled": lambda: small_variant("longctx_paged_tree16"),        # G = 8, T = 16
    "d64_bs8": lambda: small_variant("sparse_topk32_ctx64k", D=64, bs=8, ctx_lo=37, ctx_hi=90),
    "tree64_g4": lambda: small_variant("llama3_8b_tree64", topk=7),            # 256 rows per group
    "ragged_short": lambda: small_variant("sparse_topk32_ctx64k", B=3, ctx_lo=1, ctx_hi=200, topk=9, hot_blocks=1),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_shared_selection_matches_oracle(case):
    c = CASES[case]()
    _say("shared top-k %s" % case)
    x = make_inputs(c)
    d = to_device(x)
    k = c.topk or 4
    ref = oracle.topk_blocks_shared(x.q, x.k_pages, x.block_table, x.ctx_lens, c.bs, k, c.dtype)
    a = tva.topk_blocks_shared(d["q"], d["k"], d["table"], d["ctx"], k)
    sums = tva.block_sums(d["k"], d["table"], d["ctx"])
    b = tva.topk_blocks_shared(d["q"], d["k"], d["table"], d["ctx"], k, sums=sums)
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    assert np.array_equal(a.cpu().numpy(), ref)
    assert np.array_equal(b.cpu().numpy(), ref)


@pytest.mark.parametrize("k", [1, 64, 2000])
def test_shared_selection_edge_k(k):
    """k = 1, k at the attention's limit, and k above the block count (every
    block kept, -1 padded)."""
    c = small_variant("sparse_topk32_ctx64k", B=2, ctx_lo=900, ctx_hi=1500)
    _say("shared top-k k=%d" % k)
    x = make_inputs(c)
    d = to_device(x)
    ref = oracle.topk_blocks_shared(x.q, x.k_pages, x.block_table, x.ctx_lens, c.bs, k, c.dtype)
    got = tva.topk_blocks_shared(d["q"], d["k"], d["table"], d["ctx"], k)
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    assert np.array_equal(got.cpu().numpy(), ref)


def test_shared_selection_full_size():
    """Full 4 x 64K context with kept sums, the call the sparse step times."""
    c = CONFIGS["sparse_topk32_ctx64k"]
    _say("shared top-k full size")
    x = make_inputs(c)
    d = to_device(x)
    sums = tva.block_sums(d["k"], d["table"], d["ctx"])
    got = tva.topk_blocks_shared(d["q"], d["k"], d["table"], d["ctx"], c.topk, sums=sums)
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    ref = oracle.topk_blocks_shared(x.q, x.k_pages, x.block_table, x.ctx_lens, c.bs, c.topk, c.dtype)
    assert np.array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("size", ["small", "full"])
def test_sparse_attention_over_shared_selection(size):
    name = "sparse_topk32_ctx64k"
    c = small_variant(name) if size == "small" else CONFIGS[name]
    _say("sparse attention shared %s" % size)
    x = make_inputs(c)
    d = to_device(x)
    sel = tva.topk_blocks_shared(d["q"], d["k"], d["table"], d["ctx"], c.topk)
    out = tva.tree_verify_attn(d["q"], d["k"], d["v"], d["table"], d["ctx"], d["parent"], sel_blocks=sel)
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    gpu = host_f64(out)
    ref_sel = oracle.topk_blocks_shared(x.q, x.k_pages, x.block_table, x.ctx_lens, c.bs, c.topk, c.dtype)
    assert np.array_equal(sel.cpu().numpy(), ref_sel)
    if size == "small":
        ref = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens,
                                     x.tree_parent, c.bs, c.dtype, sel_blocks=ref_sel)
        check_attention(gpu, ref, c.dtype, "sparse shared small")
    else:
        r = np.random.default_rng(7)
        rows = {(int(r.integers(c.B)), int(r.integers(c.T)), int(r.integers(c.Hq))) for _ in range(24)}
        rows = sorted(rows | {(0, 0, 0), (c.B - 1, c.T - 1, c.Hq - 1)})
        ref = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens,
                                     x.tree_parent, c.bs, c.dtype, sel_blocks=ref_sel, rows=rows)
        check_attention(np.stack([gpu[b, i, h] for b, i, h in rows]), ref, c.dtype, "sparse shared full")


def test_shared_selection_workspace_reuse():
    c = small_variant("sparse_topk32_ctx64k", B=2)
    x = make_inputs(c)
    d = to_device(x)
    a = tva.topk_blocks_shared(d["q"], d["k"], d["table"], d["ctx"], 5)
    p = tva.topk_blocks(d["q"], d["k"], d["table"], d["ctx"], 5)          # same workspace, per row
    b = tva.topk_blocks_shared(d["q"], d["k"], d["table"], d["ctx"], 5)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = oracle.topk_blocks(x.q, x.k_pages, x.block_table, x.ctx_lens, c.bs, 5, c.dtype)
    assert np.array_equal(p.cpu().numpy(), ref)


def test_shared_selection_bad_block_sets_status():
    """A context block id out of range under the kept-sums path: the block
    bit is set, the call completes, and a sequence whose table is sound gets
    the oracle's list."""
    from tests.devutil import dev_tensor
    c = small_variant("sparse_topk32_ctx64k", B=2, ctx_lo=300, ctx_hi=300, hot_blocks=1)
    x = make_inputs(c)
    d = to_device(x)
    sums = tva.block_sums(d["k"], d["table"], d["ctx"])
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    table = x.block_table.copy()
    table[1, 2] = x.k_pages.shape[0] + 5
    _say("shared top-k bad block")
    sel = tva.topk_blocks_shared(d["q"], d["k"], dev_tensor(table), d["ctx"], 3, sums=sums)
    torch.cuda.synchronize()
    assert tva.device_status() & 0x2
    ref = oracle.topk_blocks_shared(x.q, x.k_pages, x.block_table, x.ctx_lens, c.bs, 3, c.dtype)
    assert np.array_equal(sel.cpu().numpy()[0], ref[0])
