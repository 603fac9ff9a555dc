"""The draft-cache recalibration pass on the GPU (EasySpec page, "Approach":
after each draft-and-verify round the drafter's cache entries for the
accepted tokens are recomputed in one token-parallel pass).  Its hot path is
chain-shaped multi-token attention over the drafter's paged cache, with the
recomputed K/V already written at slots ctx_b .. ctx_b + n_b - 1, followed by
a commit of the identity path of length n_b.  Checked against the oracle's
attention (a chain is causal attention) and commit, at a drafter's shape
(32/8 heads, D = 64) with a different accepted length per sequence."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_inputs
from tests.devutil import check_attention, host_f64, to_device

tva = pytest.importorskip("tree_verification_amd")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _drafter(B, T, ctx_lo, ctx_hi, dtype="bf16", seed=0):
    return dataclasses.replace(
        CONFIGS["llama3_8b_tree64"], name="drafter_calibration", B=B, T=T, Hq=32, Hkv=8, D=64,
        dtype=dtype, ctx_lo=ctx_lo, ctx_hi=ctx_hi, tree="chain", max_parent_depth=0, max_children=0,
        V=1024, shuffle_table=True, seed=seed)


def _host_pages(t, dtype):
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _calibrate(c, x, d, n):
    """Chain attention over the cache, then the identity-path commit of n[b]
    tokens per sequence."""
    out = tva.tree_verify_attn(d["q"], d["k"], d["v"], d["table"], d["ctx"], d["parent"])
    path = torch.arange(c.T, dtype=torch.int32, device="cuda").repeat(c.B, 1).contiguous()
    plen = torch.tensor(n, dtype=torch.int32, device="cuda")
    tva.kv_commit(d["k"], d["v"], d["table"], d["ctx"], path, plen)
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    return host_f64(out), path.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_calibration_small(dtype):
    c = _drafter(B=4, T=8, ctx_lo=90, ctx_hi=300, dtype=dtype)
    _say("calibration small %s" % dtype)
    x = make_inputs(c)
    assert (x.tree_parent[0] == np.arange(-1, c.T - 1)).all()
    n = np.random.default_rng(1).integers(1, c.T + 1, size=c.B).astype(np.int32)
    d = to_device(x)
    gpu, path = _calibrate(c, x, d, n)
    ref = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens, x.tree_parent,
                                 c.bs, c.dtype)
    for b in range(c.B):              # rows past n_b are padding; every row is still checked
        check_attention(gpu[b], ref[b], c.dtype, "calibration b=%d" % b)
    K, V, ctx2 = oracle.commit(x.k_pages, x.v_pages, x.block_table, x.ctx_lens, path, n, c.bs)
    assert np.array_equal(K.view(np.uint8), x.k_pages.view(np.uint8))   # identity path: nothing moves
    assert np.array_equal(_host_pages(d["k"], c.dtype).view(np.uint8), K.view(np.uint8))
    assert np.array_equal(_host_pages(d["v"], c.dtype).view(np.uint8), V.view(np.uint8))
    assert np.array_equal(d["ctx"].cpu().numpy(), ctx2)
    assert np.array_equal(ctx2, x.ctx_lens + n)


def test_calibration_chain_is_causal_attention():
    """Each chain row equals causal attention over context + the chain prefix,
    computed directly from the dense key/value rows."""
    c = _drafter(B=2, T=6, ctx_lo=40, ctx_hi=70, dtype="f32")
    x = make_inputs(c)
    d = to_device(x)
    gpu, _ = _calibrate(c, x, d, np.full(c.B, c.T, np.int32))
    G = c.Hq // c.Hkv
    for b in range(c.B):
        ctx = int(x.ctx_lens[b])
        rows_k = np.stack([x.k_pages[x.block_table[b, p // c.bs], :, p % c.bs] for p in range(ctx + c.T)])
        rows_v = np.stack([x.v_pages[x.block_table[b, p // c.bs], :, p % c.bs] for p in range(ctx + c.T)])
        for i in range(c.T):
            for h in range(c.Hq):
                kk = rows_k[:ctx + i + 1, h // G].astype(np.float64)
                vv = rows_v[:ctx + i + 1, h // G].astype(np.float64)
                s = kk @ x.q[b, i, h].astype(np.float64) / np.sqrt(c.D)
                p = np.exp(s - s.max())
                want = (p / p.sum()) @ vv
                assert np.abs(gpu[b, i, h] - want).max() <= 1e-5 * np.abs(want).max()


def test_calibration_full_drafter_shape():
    """B = 16 sequences of 4096 context, 8-token chains, sampled rows."""
    c = _drafter(B=16, T=8, ctx_lo=4096, ctx_hi=4096)
    _say("calibration full")
    x = make_inputs(c)
    n = np.random.default_rng(2).integers(1, c.T + 1, size=c.B).astype(np.int32)
    d = to_device(x)
    gpu, _ = _calibrate(c, x, d, n)
    r = np.random.default_rng(3)
    rows = sorted({(int(r.integers(c.B)), int(r.integers(c.T)), int(r.integers(c.Hq))) for _ in range(24)}
                  | {(0, 0, 0), (c.B - 1, c.T - 1, c.Hq - 1)})
    ref = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens, x.tree_parent,
                                 c.bs, c.dtype, rows=rows)
    check_attention(np.stack([gpu[b, i, h] for b, i, h in rows]), ref, c.dtype, "calibration full")
    assert np.array_equal(d["ctx"].cpu().numpy(), x.ctx_lens + n)
