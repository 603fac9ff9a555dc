"""Rejection sampling at wide nodes and with zero residual mass, on the GPU,
against the oracle: every sibling of a node is tested however many are
rejected before it, and a rejection that leaves no residual mass keeps the
target as it was (reading R9)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth.inputs import f32_to_bf16_bits
from tests.devutil import compare_accept, dev_tensor

tva = pytest.importorskip("tree_verification_amd")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _unif(rng, shape):
    return (rng.integers(0, 1 << 24, size=shape) * 2.0 ** -24).astype(np.float32)


def _run(logits, ldt, qd, parent, tok, unif, tau):
    """GPU acceptance and the oracle's on the same arrays; exact compare up to
    near ties at the decisive event.  Returns the GPU results."""
    d = [dev_tensor(a) for a in (logits, qd, parent, tok, unif)]
    p, l, b = tva.accept(d[0], d[1], d[2], d[3], d[4], tau)
    torch.cuda.synchronize()
    gpu = (p.cpu().numpy(), l.cpu().numpy(), b.cpu().numpy())
    assert tva.device_status() == 0
    ref = oracle.accept(logits, ldt, qd, parent, tok, unif, tau, trace=True)
    compare_accept(gpu, ref[:3], ref[3])
    return gpu, ref


def _wide_closed_form(B, V, ldt, seed):
    """Root with 100 children: 99 carry token 0, the last token 3 (or 0 too
    in every other sequence).  p = 1/V (zero logits), q(0) = 0.9, q(y) =
    0.1/(V-1) elsewhere: the first child is rejected, the residual is then
    uniform over tokens 1..V-1 and r(0) = 0 rejects children 2..99, so the
    walk tests all 100 and takes child 100 when it carries token 3; else the
    bonus comes from the uniform residual."""
    rng = np.random.default_rng(seed)
    n = 100
    T = n + 1
    parent = np.array([[-1] + [0] * n], np.int32)
    tok = np.zeros((B, T), np.int32)
    tok[:, 100] = np.where(np.arange(B) % 2 == 0, 3, 0)
    parent = np.repeat(parent, B, axis=0)
    lg = np.zeros((B, T, V), np.float32)
    logits = f32_to_bf16_bits(lg) if ldt == "bf16" else lg
    q = np.full(V, 0.1 / (V - 1), np.float32)
    q[0] = 0.9
    qd = np.ascontiguousarray(np.broadcast_to(q, (B, T, V)))
    unif = _unif(rng, (B, T, 2))
    unif[:, 1, 0] = np.maximum(unif[:, 1, 0], 0.25)   # u q(0) >= 0.225 > 1/V: rejected
    return logits, qd, parent, tok, unif


@pytest.mark.parametrize("V,ldt", [(16, "f32"), (16, "bf16"), (32000, "bf16"), (32000, "f32")])
def test_wide_node_closed_form(V, ldt):
    B = 64 if V < 10000 else 32          # 1 and 8 workgroups per sequence
    _say("accept wide closed form V=%d %s B=%d" % (V, ldt, B))
    logits, qd, parent, tok, unif = _wide_closed_form(B, V, ldt, seed=V)
    (gp, gl, gb), _ = _run(logits, ldt, qd, parent, tok, unif, 1.0)
    even = np.arange(B) % 2 == 0
    assert np.all(gl[even] == 2) and np.all(gp[even, 1] == 100)
    assert np.all(gl[~even] == 1) and np.all(gb[~even] != 0)


def _peaked_wide(B, V, n_kids, ldt, tau, seed, grand=3):
    """One node with n_kids i.i.d. siblings from a drafter peaked on one token
    (its logit 6 + 0.8 log(V / 16) above N(0, 1) noise, so that its
    probability is about the same for every V), target logits N(0, 1); each of the root's
    children has `grand` children of its own, so the walk goes on below the
    wide node."""
    rng = np.random.default_rng(seed)
    T = 1 + n_kids + grand * n_kids
    par = np.zeros(T, np.int32)
    par[0] = -1
    par[1:1 + n_kids] = 0
    par[1 + n_kids:] = 1 + np.repeat(np.arange(n_kids), grand)
    parent = np.repeat(par[None], B, axis=0)
    draft_l = rng.standard_normal((B, T, V)).astype(np.float64)
    draft_l[:, :, 5] += 6.0 + 0.8 * np.log(V / 16.0)
    q = np.exp(draft_l / tau - (draft_l / tau).max(-1, keepdims=True))
    q = (q / q.sum(-1, keepdims=True)).astype(np.float32)
    qd = q / q.sum(-1, keepdims=True, dtype=np.float64).astype(np.float32)
    tok = np.zeros((B, T), np.int32)
    qq = q.astype(np.float64)
    for b in range(B):
        for i in range(1, T):
            w = qq[b, par[i]]
            tok[b, i] = rng.choice(V, p=w / w.sum())
    lg = rng.standard_normal((B, T, V)).astype(np.float32)
    logits = f32_to_bf16_bits(lg) if ldt == "bf16" else lg
    unif = _unif(rng, (B, T, 2))
    return logits, np.ascontiguousarray(qd), parent, tok, unif


@pytest.mark.parametrize("V,ldt,n_kids,grand", [(16, "bf16", 100, 3), (16, "f32", 128, 3),
                                                (4096, "bf16", 100, 3), (8192, "f32", 100, 0)])
def test_wide_node_peaked_drafter(V, ldt, n_kids, grand):
    """B = 64 sequences (1, 2 and 4 workgroups per sequence); many walks
    test more than 64 siblings of the root before one is accepted or all are
    rejected."""
    B, tau = 64, 0.8
    _say("accept wide peaked V=%d %s kids=%d" % (V, ldt, n_kids))
    logits, qd, parent, tok, unif = _peaked_wide(B, V, n_kids, ldt, tau, seed=100 + V, grand=grand)
    (gp, gl, gb), (rp, rl, rb, ev) = _run(logits, ldt, qd, parent, tok, unif, tau)
    # the case reaches what it is for: walks that test more than 64 siblings
    tests_at_root = [sum(1 for e in evs if e[0] == "test" and e[1] == 0) for evs in ev]
    assert max(tests_at_root) > 64
    assert any(rl[b] > 1 and rp[b, 1] > 64 for b in range(B))


@pytest.mark.parametrize("V,ldt", [(8, "f32"), (8, "bf16"), (32000, "bf16"), (32000, "f32")])
def test_zero_residual_mass(V, ldt):
    """q = 2p everywhere (a draft row summing to 2): a rejection leaves no
    residual mass, the target stays p = 1/V, and child c is accepted iff
    u_c < 1/2; with every child rejected the bonus comes from p."""
    B = 64 if V < 10000 else 32
    _say("accept zero residual V=%d %s" % (V, ldt))
    rng = np.random.default_rng(7 + V)
    n = 12
    T = n + 1
    parent = np.repeat(np.array([[-1] + [0] * n], np.int32), B, axis=0)
    tok = rng.integers(0, V, size=(B, T)).astype(np.int32)
    lg = np.zeros((B, T, V), np.float32)
    logits = f32_to_bf16_bits(lg) if ldt == "bf16" else lg
    qd = np.full((B, T, V), 2.0 / V, np.float32)
    unif = _unif(rng, (B, T, 2))
    unif[:, 1:, 0] = 0.5 + 0.5 * unif[:, 1:, 0]                    # reject ...
    pick = rng.integers(1, n + 1, size=B)
    for b in range(0, B, 2):                                          # ... except one child in half
        unif[b, pick[b], 0] = 0.25
    (gp, gl, gb), _ = _run(logits, ldt, qd, parent, tok, unif, 1.0)
    for b in range(B):
        if b % 2 == 0:
            assert gl[b] == 2 and gp[b, 1] == pick[b]
        else:
            assert gl[b] == 1
            uv = float(unif[b, 0, 1]) * V
            if abs(uv - round(uv)) > 1e-6:       # (off an exact CDF boundary)
                assert gb[b] == int(uv)
