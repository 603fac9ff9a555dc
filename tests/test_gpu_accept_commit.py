"""sd_accept_commit on the GPU: the acceptance walk and the commit of its
paths in one launch, against the oracle's accept and commit (and against the
two separate calls), including the error paths."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_inputs, small_variant
from synth.configs import CONFIG_ORDER
from tests.devutil import compare_accept, dev_tensor, to_device

tva = pytest.importorskip("tree_verification_amd")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _tau(c):
    return 0.0 if c.mode == "greedy" else c.temperature


def _host_pages(t, dtype):
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _fused(c, d):
    tau = _tau(c)
    draft = d["draft"] if c.mode == "mss" else None
    p, l, b = tva.accept_commit(d["logits"], draft, d["parent"], d["token"], d["unif"], tau,
                                d["k"], d["v"], d["table"], d["ctx"])
    torch.cuda.synchronize()
    return p.cpu().numpy(), l.cpu().numpy(), b.cpu().numpy()


def _check_against_oracle(c, x, d, gpu):
    tau = _tau(c)
    ref = oracle.accept(x.target_logits, c.logit_dtype, x.draft_probs if c.mode == "mss" else None,
                        x.tree_parent, x.tree_token, x.uniforms, tau, trace=True)
    compare_accept(gpu, ref[:3], ref[3])
    # the cache and lengths follow the oracle's commit of the path the GPU took
    K, V, ctx2 = oracle.commit(x.k_pages, x.v_pages, x.block_table, x.ctx_lens, gpu[0], gpu[1], c.bs)
    assert np.array_equal(_host_pages(d["k"], c.dtype).view(np.uint8), K.view(np.uint8))
    assert np.array_equal(_host_pages(d["v"], c.dtype).view(np.uint8), V.view(np.uint8))
    assert np.array_equal(d["ctx"].cpu().numpy(), ctx2)


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_accept_commit_small(name):
    c = small_variant(name)
    _say("accept_commit small %s" % name)
    x = make_inputs(c)
    d = to_device(x)
    gpu = _fused(c, d)
    assert tva.device_status() == 0
    _check_against_oracle(c, x, d, gpu)


@pytest.mark.parametrize("name", ["llama3_8b_tree64", "specexec_70b_tree2048"])
def test_accept_commit_full_size(name):
    """Full sizes: the launch bench.py times (16 workgroups per sequence over
    8 KV heads), and the 2048-node tree."""
    c = CONFIGS[name]
    _say("accept_commit full %s" % name)
    x = make_inputs(c)
    d = to_device(x)
    gpu = _fused(c, d)
    assert tva.device_status() == 0
    _check_against_oracle(c, x, d, gpu)


def test_accept_commit_equals_two_calls():
    c = CONFIGS["llama3_8b_tree64"]
    _say("accept_commit vs accept + kv_commit")
    x = make_inputs(c)
    d1, d2 = to_device(x), to_device(x)
    tau = _tau(c)
    p, l, b = tva.accept(d1["logits"], d1["draft"], d1["parent"], d1["token"], d1["unif"], tau)
    tva.kv_commit(d1["k"], d1["v"], d1["table"], d1["ctx"], p, l)
    gpu = _fused(c, d2)
    assert tva.device_status() == 0
    assert np.array_equal(gpu[0], p.cpu().numpy())
    assert np.array_equal(gpu[1], l.cpu().numpy())
    assert np.array_equal(gpu[2], b.cpu().numpy())
    for key in ("k", "v", "ctx"):
        assert torch.equal(d1[key], d2[key]), key


@pytest.mark.parametrize("V", [1000, 8192, 40000])
def test_accept_commit_heads_per_workgroup(V):
    """Vocabulary sizes that give 1, 4 and 16 workgroups per sequence over 8
    KV heads: one workgroup copies all heads, two heads each, or one head
    each with the rest idle."""
    c = small_variant("llama3_8b_tree64", B=4, T=24, V=V, ctx_lo=37, ctx_hi=90)
    _say("accept_commit V=%d" % V)
    x = make_inputs(c)
    d = to_device(x)
    gpu = _fused(c, d)
    assert tva.device_status() == 0
    _check_against_oracle(c, x, d, gpu)


@pytest.mark.parametrize("mode", ["greedy", "exec"])
def test_accept_commit_other_rules(mode):
    c = dataclasses.replace(small_variant("llama3_8b_tree64", B=3, T=32), mode=mode,
                            temperature=0.0 if mode == "greedy" else 0.7)
    _say("accept_commit %s" % mode)
    x = make_inputs(c)
    d = to_device(x)
    gpu = _fused(c, d)
    assert tva.device_status() == 0
    _check_against_oracle(c, x, d, gpu)


def test_accept_commit_bad_block_leaves_sequence():
    """A block of sequence 1's tree slots out of range: its path is still
    returned, its cache and length are left as they were, the block bit is
    set; sequence 0 commits normally."""
    c = small_variant("llama3_8b_tree64", B=2, T=8, ctx_lo=40, ctx_hi=40)
    x = make_inputs(c)
    x.block_table[1, 40 // c.bs] = x.k_pages.shape[0] + 3
    d = to_device(x)
    _say("accept_commit bad block")
    gpu = _fused(c, d)
    assert tva.device_status() & 0x2
    ref = oracle.accept(x.target_logits, c.logit_dtype, x.draft_probs, x.tree_parent, x.tree_token,
                        x.uniforms, _tau(c), trace=True)
    compare_accept(gpu, ref[:3], ref[3])
    plen = gpu[1].copy()
    plen[1] = 0                                  # sequence 1 commits nothing
    K, V, ctx2 = oracle.commit(x.k_pages, x.v_pages, x.block_table, x.ctx_lens, gpu[0], plen, c.bs)
    assert np.array_equal(_host_pages(d["k"], c.dtype), K)
    assert np.array_equal(_host_pages(d["v"], c.dtype), V)
    assert d["ctx"].cpu().tolist() == [int(ctx2[0]), int(x.ctx_lens[1])]


def test_accept_commit_bad_tree_commits_nothing():
    c = small_variant("llama3_8b_tree64", B=2, T=8, ctx_lo=40, ctx_hi=40)
    x = make_inputs(c)
    x.tree_parent[0, 5] = 6                      # sequence 0's tree points forward
    d = to_device(x)
    _say("accept_commit bad tree")
    k0, v0 = d["k"].clone(), d["v"].clone()
    gpu = _fused(c, d)
    assert tva.device_status() & 0x1
    assert gpu[1][0] == 0 and gpu[2][0] == -1
    assert int(d["ctx"][0]) == int(x.ctx_lens[0])
    # sequence 1 is committed as usual
    ref = oracle.accept(x.target_logits[1:], c.logit_dtype, x.draft_probs[1:], x.tree_parent[1:],
                        x.tree_token[1:], x.uniforms[1:], _tau(c), trace=True)
    compare_accept(tuple(g[1:] for g in gpu), ref[:3], ref[3])
    plen = gpu[1].copy()
    plen[0] = 0
    K, V, ctx2 = oracle.commit(x.k_pages, x.v_pages, x.block_table, x.ctx_lens, gpu[0], plen, c.bs)
    assert np.array_equal(_host_pages(d["k"], c.dtype), K)
    assert np.array_equal(_host_pages(d["v"], c.dtype), V)
    assert int(d["ctx"][1]) == int(ctx2[1])
    del k0, v0
