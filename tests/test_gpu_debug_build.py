"""The debug build (libsdtree_debug.so, the kernels compiled with their
device-side consistency checks) on representative calls: dense, split and
sparse attention, the acceptance walk with its commit, block selection, the
shared selection and the tree build.  Every call must leave the debug bit
clear, and its results must equal the release library's on the same inputs
(the checks add no arithmetic)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_inputs, small_variant
from synth.inputs import _normals, _rng, S_DRAFT
from tests.devutil import dev_tensor, to_device

tva = pytest.importorskip("tree_verification_amd")
from tree_verification_amd import _lib  # noqa: E402

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _host(t):
    if isinstance(t, torch.Tensor):
        # (bf16 compared as its bit patterns)
        return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).cpu().numpy()
    return np.asarray(t)


def _both(fn):
    """fn() run on the release and on the debug library; returns both results
    as host arrays, after checking that the debug calls set no status bit."""
    out = []
    for path in (_lib.LIB_PATH, _lib.DEBUG_LIB_PATH):
        prev = _lib.use_library(path)
        try:
            r = fn()
            torch.cuda.synchronize()
            bits = tva.device_status()
        finally:
            _lib.use_library(prev)
        assert bits == 0, "%s: status bits 0x%x" % (path, bits)
        out.append([_host(t) for t in r])
    return out


def _same(rel, dbg, what):
    for a, b in zip(rel, dbg):
        assert a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8)), what


@pytest.mark.parametrize("name", ["llama3_8b_tree64", "longctx_paged_tree16", "specexec_70b_tree2048"])
def test_debug_attention_equals_release(name):
    """Dense attention (two query tiles per KV head; context splits; the
    256-row tiles of a large tree)."""
    c = small_variant(name)
    _say("debug attention %s" % name)
    x = make_inputs(c)
    d = to_device(x)
    rel, dbg = _both(lambda: [tva.tree_verify_attn(d["q"], d["k"], d["v"], d["table"], d["ctx"], d["parent"])])
    _same(rel, dbg, name)


@pytest.mark.parametrize("k,dtype", [(6, "bf16"), (150, "bf16"), (150, "f32")])
def test_debug_sparse_attention_and_topk_equal_release(k, dtype):
    c = small_variant("sparse_topk32_ctx64k", topk=k, dtype=dtype, bs=8, ctx_lo=1500, ctx_hi=2500, B=2)
    _say("debug sparse k=%d %s" % (k, dtype))
    x = make_inputs(c)
    d = to_device(x)

    def run():
        sel = tva.topk_blocks(d["q"], d["k"], d["table"], d["ctx"], k)
        out = tva.tree_verify_attn(d["q"], d["k"], d["v"], d["table"], d["ctx"], d["parent"], sel_blocks=sel)
        shared = tva.topk_blocks_shared(d["q"], d["k"], d["table"], d["ctx"], k)
        return [sel, out, shared]
    rel, dbg = _both(run)
    _same(rel, dbg, "sparse k=%d" % k)


def test_debug_accept_commit_equals_release():
    c = small_variant("llama3_8b_tree64")
    _say("debug accept+commit")
    x = make_inputs(c)

    def run():
        d = to_device(x)
        p, l, b = tva.accept_commit(d["logits"], d["draft"], d["parent"], d["token"], d["unif"],
                                    c.temperature, d["k"], d["v"], d["table"], d["ctx"])
        return [p, l, b, d["k"], d["v"], d["ctx"]]
    rel, dbg = _both(run)
    _same(rel, dbg, "accept+commit")
    # and the walk is the oracle's
    r = oracle.accept(x.target_logits, c.logit_dtype, x.draft_probs, x.tree_parent, x.tree_token,
                      x.uniforms, c.temperature)
    assert np.array_equal(rel[1], r[1])


def test_debug_tree_build_equals_release():
    c = CONFIGS["specexec_70b_tree2048"]
    _say("debug tree build 160 x 4099")
    dr = _normals(_rng(c, S_DRAFT), (160, 4099), c.logit_sigma, "f32")
    rel, dbg = _both(lambda: list(tva.tree_build(dev_tensor(dr), 1.0, 0)[:3]))
    _same(rel, dbg, "tree build")
