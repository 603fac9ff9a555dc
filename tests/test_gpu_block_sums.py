"""Kept block key sums on the GPU (sd_block_sums, sd_block_sums_append,
sd_topk_blocks_cached) against the oracle: the sums bit for bit, the
cached selection equal to the selection read from K, and the sums extended
after a commit equal to sums rebuilt at the new lengths."""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_inputs, small_variant
from tests.devutil import dev_tensor, to_device

tva = pytest.importorskip("tree_verification_amd")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _live(ctx_lens, table, bs):
    """Physical blocks holding context of some sequence."""
    used = set()
    for b in range(len(ctx_lens)):
        for n in range((int(ctx_lens[b]) + bs - 1) // bs):
            used.add(int(table[b, n]))
    return sorted(used)


def _check_sums(got, ref, blocks):
    g = got.cpu().numpy()
    assert np.array_equal(g[blocks].view(np.uint32), ref[blocks].view(np.uint32))


CASES = {
    "sparse_small": lambda: small_variant("sparse_topk32_ctx64k"),
    "sparse_small_f32": lambda: small_variant("sparse_topk32_ctx64k", dtype="f32"),
    "longctx_shuffled": lambda: small_variant("longctx_paged_tree16"),
    "d64_bs8": lambda: small_variant("sparse_topk32_ctx64k", D=64, bs=8, ctx_lo=37, ctx_hi=90),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_block_sums_and_cached_topk_match_oracle(case):
    c = CASES[case]()
    _say("block sums %s" % case)
    x = make_inputs(c)
    d = to_device(x)
    sums = tva.block_sums(d["k"], d["table"], d["ctx"])
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    ref = oracle.block_sums(x.k_pages, x.block_table, x.ctx_lens, c.bs, c.dtype)
    _check_sums(sums, ref, _live(x.ctx_lens, x.block_table, c.bs))
    k = c.topk or 4
    sel = tva.topk_blocks_cached(d["q"], sums, d["k"], d["table"], d["ctx"], k)
    rsel = oracle.topk_blocks(x.q, x.k_pages, x.block_table, x.ctx_lens, c.bs, k, c.dtype)
    assert np.array_equal(sel.cpu().numpy(), rsel)


def test_cached_topk_full_size_equals_topk_from_k():
    """Full C5 (4 x 64K context, 1024 blocks per sequence): the cached
    selection equals the selection formed from K (itself pinned to the
    oracle at this size by the top-k parity test)."""
    c = CONFIGS["sparse_topk32_ctx64k"]
    _say("cached top-k full size")
    x = make_inputs(c)
    d = to_device(x)
    sums = tva.block_sums(d["k"], d["table"], d["ctx"])
    a = tva.topk_blocks(d["q"], d["k"], d["table"], d["ctx"], c.topk)
    b = tva.topk_blocks_cached(d["q"], sums, d["k"], d["table"], d["ctx"], c.topk)
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    assert torch.equal(a, b)
    # sampled blocks against the oracle's sums
    rng = np.random.default_rng(3)
    blocks = sorted(rng.choice(_live(x.ctx_lens, x.block_table, c.bs), size=24, replace=False).tolist())
    for blk in blocks:
        b_, n_ = np.argwhere(x.block_table == blk)[0]
        valid = min(c.bs, int(x.ctx_lens[b_]) - int(n_) * c.bs)
        ref = oracle.topk._block_sum(x.k_pages, blk, 0, valid, c.dtype)
        assert np.array_equal(sums[blk].cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("ctx0", [128, 125, 61, 3])
def test_block_sums_append_after_commit(ctx0):
    """Sums kept through a commit (acceptance and commit in one launch, then
    the append) equal sums rebuilt at the new lengths, and the cached
    selection at the new lengths equals the oracle's: the appended positions
    start a new block (128), cross a block boundary (125, 61), or extend a
    short context (3)."""
    c = small_variant("sparse_topk32_ctx64k", B=3, ctx_lo=ctx0, ctx_hi=ctx0 + 2, hot_blocks=1)
    _say("block sums append ctx0=%d" % ctx0)
    x = make_inputs(c)
    d = to_device(x)
    sums = tva.block_sums(d["k"], d["table"], d["ctx"])
    p, l, b = tva.accept_commit(d["logits"], None, d["parent"], d["token"], d["unif"], 0.0,
                                d["k"], d["v"], d["table"], d["ctx"])
    tva.block_sums_append(d["k"], d["table"], d["ctx"], l, sums)
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    plen = l.cpu().numpy()
    K, V, ctx2 = oracle.commit(x.k_pages, x.v_pages, x.block_table, x.ctx_lens, p.cpu().numpy(), plen,
                               c.bs)
    assert np.array_equal(d["ctx"].cpu().numpy(), ctx2)
    ref = oracle.block_sums(K, x.block_table, ctx2, c.bs, c.dtype)
    live = _live(ctx2, x.block_table, c.bs)
    _check_sums(sums, ref, live)
    # the oracle's own extension agrees
    ext = oracle.append_block_sums(oracle.block_sums(x.k_pages, x.block_table, x.ctx_lens, c.bs, c.dtype),
                                   K, x.block_table, ctx2, plen, c.bs, c.dtype)
    assert np.array_equal(ext[live].view(np.uint32), ref[live].view(np.uint32))
    sel = tva.topk_blocks_cached(d["q"], sums, d["k"], d["table"], d["ctx"], c.topk)
    rsel = oracle.topk_blocks(x.q, K, x.block_table, ctx2, c.bs, c.topk, c.dtype)
    assert np.array_equal(sel.cpu().numpy(), rsel)


def test_block_sums_append_bad_block_leaves_sums():
    c = small_variant("sparse_topk32_ctx64k", B=2, ctx_lo=100, ctx_hi=100, hot_blocks=1)
    x = make_inputs(c)
    d = to_device(x)
    sums = tva.block_sums(d["k"], d["table"], d["ctx"])
    before = sums.clone()
    table = x.block_table.copy()
    table[1, 110 // c.bs] = x.k_pages.shape[0] + 7          # the block position 100..109 reaches
    ctx_new = dev_tensor(np.array([104, 110], np.int32))
    n_new = dev_tensor(np.array([4, 10], np.int32))
    _say("block sums append bad block")
    tva.block_sums_append(d["k"], dev_tensor(table), ctx_new, n_new, sums)
    torch.cuda.synchronize()
    assert tva.device_status() & 0x2
    ref = oracle.append_block_sums(before.cpu().numpy(), x.k_pages, table, np.array([104, 100], np.int32),
                                   np.array([4, 0], np.int32), c.bs, c.dtype)
    got = sums.cpu().numpy()
    blk0 = int(table[0, 100 // c.bs])
    assert np.array_equal(got[blk0].view(np.uint32), ref[blk0].view(np.uint32))
    # sequence 1 is untouched
    mask = np.ones(got.shape[0], bool)
    mask[blk0] = False
    assert np.array_equal(got[mask].view(np.uint32), before.cpu().numpy()[mask].view(np.uint32))


@pytest.mark.parametrize("ctx0,case", [(128, "bf16"), (125, "bf16"), (61, "f32"), (3, "bf16"),
                                       (37, "d64_bs8")])
@pytest.mark.parametrize("call", ["accept_commit", "kv_commit", "noalloc"])
def test_commit_extends_sums_in_the_same_launch(ctx0, case, call):
    """The kept sums passed to the commit (sd_accept_commit, sd_kv_commit or
    the no-workspace variant) come out equal to sums rebuilt at the new
    lengths, bit for bit, and equal to the separate append's."""
    over = dict(B=3, ctx_lo=ctx0, ctx_hi=ctx0 + 2, hot_blocks=1)
    if case == "f32":
        over["dtype"] = "f32"
    if case == "d64_bs8":
        over.update(D=64, bs=8)
    c = small_variant("sparse_topk32_ctx64k", **over)
    _say("commit with sums %s ctx0=%d %s" % (call, ctx0, case))
    x = make_inputs(c)
    d = to_device(x)
    sums = tva.block_sums(d["k"], d["table"], d["ctx"])
    sums_sep = sums.clone()
    if call == "kv_commit":
        rp, rl, _ = oracle.accept(x.target_logits, c.logit_dtype, None, x.tree_parent, x.tree_token,
                                  x.uniforms, 0.0)
        p, l = dev_tensor(rp), dev_tensor(rl)
        tva.kv_commit(d["k"], d["v"], d["table"], d["ctx"], p, l, sums=sums)
    elif call == "accept_commit":
        p, l, _ = tva.accept_commit(d["logits"], None, d["parent"], d["token"], d["unif"], 0.0,
                                    d["k"], d["v"], d["table"], d["ctx"], sums=sums)
    else:
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        p, l, _ = tva.accept_commit_noalloc(d["logits"], None, d["parent"], d["token"], d["unif"], 0.0,
                                            d["k"], d["v"], d["table"], d["ctx"], status, sums=sums)
        torch.cuda.synchronize()
        assert tva.device_status(ws=status) == 0
    tva.block_sums_append(d["k"], d["table"], d["ctx"], l, sums_sep)
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    plen = l.cpu().numpy()
    K, V, ctx2 = oracle.commit(x.k_pages, x.v_pages, x.block_table, x.ctx_lens, p.cpu().numpy(), plen,
                               c.bs)
    assert np.array_equal(d["ctx"].cpu().numpy(), ctx2)
    ref = oracle.block_sums(K, x.block_table, ctx2, c.bs, c.dtype)
    live = _live(ctx2, x.block_table, c.bs)
    _check_sums(sums, ref, live)
    assert torch.equal(sums, sums_sep)
