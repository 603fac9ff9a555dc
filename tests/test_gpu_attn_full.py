"""Full-size attention checks that can fail on a mask error.

At every bf16 workload's full size, in the launch configuration bench.py
times:
  * every row of two whole (sequence, KV head) units is compared with the
    oracle (the first and the last unit, so the largest block offsets and the
    last context split are covered);
  * a planted tree makes every output depend on the mask at O(1): all query
    rows are 8 e_0, the key of every tree slot is 40 e_0 and its value a
    one-hot row (dimension (j + 7 g) mod D for slot j of KV head g), so node
    i's output is, to within 1e-6, the mean of those rows over its own
    ancestors.  A leaked key or a dropped ancestor moves an output by about
    1 / (depth + 2), 0.1 or more at these trees' depths, far past the 2e-2
    bf16 tolerance; the context's weight is below 1e-6 (its scores are at
    most about 3, the tree's 28.3)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_inputs
from synth.inputs import f32_to_bf16_bits
from tests.devutil import check_attention, dev_tensor, host_f64, to_device

tva = pytest.importorskip("tree_verification_amd")
pytestmark = pytest.mark.gpu

BF16_FULL = ["llama3_8b_tree64", "specexec_70b_tree2048", "longctx_paged_tree16",
             "sparse_topk32_ctx64k"]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _ancestors(par, i):
    out = [i]
    while par[out[-1]] >= 0:
        out.append(int(par[out[-1]]))
    return out


def _onehot_dim(j, g, D):
    return (j + 7 * g) % D


def _plant(c, x):
    """The planted tree of the module docstring, written into x's q and the
    tree slots' K/V (bf16 bit patterns); the context is left as it was."""
    B, T, Hq, D = x.q.shape
    Hkv, bs = c.Hkv, c.bs
    e0 = np.zeros(D, np.float32)
    e0[0] = 8.0
    x.q[:] = f32_to_bf16_bits(e0)[None, None, None, :]
    one = int(f32_to_bf16_bits(np.array([1.0], np.float32))[0])
    for b in range(B):
        par = x.tree_parent[0 if x.tree_parent.shape[0] == 1 else b]
        ctx = int(x.ctx_lens[b])
        krow = np.zeros(D, np.float32)
        krow[0] = 40.0
        for j in range(T):
            p = ctx + j
            blk, off = int(x.block_table[b, p // bs]), p % bs
            x.k_pages[blk, :, off, :] = f32_to_bf16_bits(krow)[None, :]
            for g in range(Hkv):
                x.v_pages[blk, g, off, :] = 0
                x.v_pages[blk, g, off, _onehot_dim(j, g, D)] = one


def _planted_expected(c, x):
    B, T, Hq, D = x.q.shape
    G = Hq // c.Hkv
    out = np.zeros((B, T, Hq, D))
    for b in range(B):
        par = x.tree_parent[0 if x.tree_parent.shape[0] == 1 else b]
        for i in range(T):
            anc = _ancestors(par, i)
            for g in range(c.Hkv):
                row = np.zeros(D)
                for j in anc:
                    row[_onehot_dim(j, g, D)] += 1.0 / len(anc)
                out[b, i, g * G:(g + 1) * G] = row
    return out


def _random_selection(c, x, seed):
    """A valid per-query selection (k ascending distinct context blocks)."""
    r = np.random.default_rng(seed)
    B, T, Hq, _ = x.q.shape
    sel = np.full((B, T, Hq, c.topk), -1, np.int32)
    for b in range(B):
        nblk = (int(x.ctx_lens[b]) + c.bs - 1) // c.bs
        for i in range(T):
            for h in range(Hq):
                k = min(c.topk, nblk)
                sel[b, i, h, :k] = np.sort(r.choice(nblk, size=k, replace=False))
    return sel


@pytest.mark.parametrize("name", BF16_FULL)
def test_attention_full_size_whole_units_and_planted_tree(name):
    c = CONFIGS[name]
    _say("attention full %s: generating" % name)
    x = make_inputs(c)
    B, T, Hq, D = x.q.shape
    G = Hq // c.Hkv
    d = to_device(x)
    _say("attention full %s: whole units" % name)
    out = tva.tree_verify_attn(d["q"], d["k"], d["v"], d["table"], d["ctx"], d["parent"])
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    gpu = host_f64(out)
    for (b, g) in [(0, 0), (B - 1, c.Hkv - 1)]:
        rows = [(b, i, h) for i in range(T) for h in range(g * G, (g + 1) * G)]
        ref = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens,
                                     x.tree_parent, c.bs, c.dtype, rows=rows)
        got = np.stack([gpu[r] for r in rows])
        check_attention(got, ref, c.dtype, "%s unit (%d, %d)" % (name, b, g))
    del d, out
    torch.cuda.empty_cache()

    _say("attention full %s: planted tree" % name)
    _plant(c, x)
    exp = _planted_expected(c, x)
    d = to_device(x)
    sels = [None] if not c.topk else [None, _random_selection(c, x, 5)]
    for sel in sels:
        out = tva.tree_verify_attn(d["q"], d["k"], d["v"], d["table"], d["ctx"], d["parent"],
                                   sel_blocks=None if sel is None else dev_tensor(sel))
        torch.cuda.synchronize()
        assert tva.device_status() == 0
        check_attention(host_f64(out), exp, c.dtype,
                        "%s planted tree%s" % (name, "" if sel is None else " (sparse)"))
