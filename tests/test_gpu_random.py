"""Seeded random sweep on the GPU: small random trees, head counts, head dims,
block sizes, ragged context lengths and shuffled block tables, in bf16 and
float32; attention (every row), acceptance (greedy and rejection sampling)
and commit against the oracle on each."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import make_inputs, small_variant
from tests.devutil import check_attention, compare_accept, dev_tensor, host_f64, to_device

tva = pytest.importorskip("tree_verification_amd")
pytestmark = pytest.mark.gpu

N_CASES = 24


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(seed):
    r = np.random.default_rng(1000 + seed)
    Hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 2, 4, 8]))
    dtype = "f32" if r.random() < 0.25 else "bf16"
    bs = int(r.choice([8, 16, 32, 64]))
    T = int(r.integers(1, 97))
    lo = int(r.integers(0, 300))
    mode = str(r.choice(["greedy", "mss"]))
    depth, kids = int(r.integers(1, 9)), int(r.integers(2, 6))
    # the random tree needs room: nodes of depth <= depth with kids - 1 children each
    while sum((kids - 1) ** k for k in range(depth + 1)) < T:
        depth, kids = depth + 1, kids + 1
    c = small_variant("llama3_8b_tree64", B=int(r.integers(1, 5)), Hq=Hkv * G, Hkv=Hkv,
                      D=int(r.choice([64, 128])), dtype=dtype, ctx_lo=lo, ctx_hi=lo + int(r.integers(0, 200)),
                      bs=bs, T=T, max_parent_depth=depth, max_children=kids,
                      V=int(r.integers(50, 3000)), logit_dtype=dtype, mode=mode,
                      temperature=float(r.choice([0.6, 0.8, 1.0])), shuffle_table=True, seed=seed)
    return c


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_case(seed):
    c = _case(seed)
    _say("random case %d: B=%d T=%d Hq/Hkv=%d/%d D=%d bs=%d ctx=[%d,%d] %s %s" % (
        seed, c.B, c.T, c.Hq, c.Hkv, c.D, c.bs, c.ctx_lo, c.ctx_hi, c.dtype, c.mode))
    x = make_inputs(c)
    d = to_device(x)
    out = tva.tree_verify_attn(d["q"], d["k"], d["v"], d["table"], d["ctx"], d["parent"])
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    ref = oracle.attention_dense(x.q, x.k_pages, x.v_pages, x.block_table, x.ctx_lens, x.tree_parent,
                                 c.bs, c.dtype)
    check_attention(host_f64(out), ref, c.dtype, "random %d" % seed)
    tau = 0.0 if c.mode == "greedy" else c.temperature
    draft = d["draft"] if c.mode == "mss" else None
    p, l, b = tva.accept_commit(d["logits"], draft, d["parent"], d["token"], d["unif"], tau,
                                d["k"], d["v"], d["table"], d["ctx"])
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    gpu = (p.cpu().numpy(), l.cpu().numpy(), b.cpu().numpy())
    r = oracle.accept(x.target_logits, c.logit_dtype, x.draft_probs if c.mode == "mss" else None,
                      x.tree_parent, x.tree_token, x.uniforms, tau, trace=True)
    compare_accept(gpu, r[:3], r[3])
    K, V, ctx2 = oracle.commit(x.k_pages, x.v_pages, x.block_table, x.ctx_lens, gpu[0], gpu[1], c.bs)
    kk = d["k"].view(torch.int16).cpu().numpy().view(np.uint16) if c.dtype == "bf16" else d["k"].cpu().numpy()
    vv = d["v"].view(torch.int16).cpu().numpy().view(np.uint16) if c.dtype == "bf16" else d["v"].cpu().numpy()
    assert np.array_equal(kk, K) and np.array_equal(vv, V)
    assert np.array_equal(d["ctx"].cpu().numpy(), ctx2)
