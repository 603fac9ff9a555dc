"""Acceptance walks that go down first-child chains longer than one round of
chained statistics (the kernel forms up to 6 chain nodes' statistics at
once), leave a chain at a node's second child, and end at a leaf, under the
three rules, with register-cached bf16 rows split over several workgroups
(and float32 rows as the uncached control); compared with the oracle on the
same arrays, exactly up to near ties at the decisive event."""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth.inputs import f32_to_bf16_bits
from tests.devutil import compare_accept, dev_tensor

tva = pytest.importorskip("tree_verification_amd")
pytestmark = pytest.mark.gpu

D = 20                                              # spine depth: 21 nodes on every path
SWITCH = [-1, 0, 2, 5, 6, 7, 12, 19]                # spine continues through the second child here


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _spine(V, ldt, rule, seed):
    """Spine node s_k (k < D) has two children, 1 + 2k and 2 + 2k (distinct
    tokens); the spine goes on through the first, or through the second at
    depth SWITCH[b].  The target logits of s_k favour the next spine node's
    token by 20 over N(0, 1) noise, so greedy takes it, target sampling draws
    it and rejection sampling accepts it (after rejecting the first child at
    the switch: the drafter gives both children 0.3).  The last spine node is
    a leaf: the walk ends with a draw (or an argmax) there."""
    rng = np.random.default_rng(seed)
    B, T = len(SWITCH), 1 + 2 * D
    parent = np.full((B, T), -1, np.int32)
    tok = np.zeros((B, T), np.int32)
    spine = np.zeros((B, D + 1), np.int64)
    for b in range(B):
        s = 0
        for k in range(D):
            a, c = 1 + 2 * k, 2 + 2 * k
            parent[b, a] = parent[b, c] = s
            tok[b, a], tok[b, c] = (7 * k + 3) % V, (7 * k + 5) % V
            s = c if k == SWITCH[b] else a
            spine[b, k + 1] = s
    lg = rng.standard_normal((B, T, V)).astype(np.float32)
    for b in range(B):
        for k in range(D):
            lg[b, spine[b, k], tok[b, spine[b, k + 1]]] += 20.0
    logits = f32_to_bf16_bits(lg) if ldt == "bf16" else lg
    qd = None
    if rule == "mss":
        q = np.full((B, T, V), 0.4 / (V - 2), np.float32)
        for b in range(B):
            for k in range(D):
                s = spine[b, k]
                q[b, s, :] = 0.4 / (V - 2)
                q[b, s, tok[b, 1 + 2 * k]] = 0.3
                q[b, s, tok[b, 2 + 2 * k]] = 0.3
        qd = q
    unif = (rng.integers(0, 1 << 24, size=(B, T, 2)) * 2.0 ** -24).astype(np.float32)
    unif[:, :, 0] = np.maximum(unif[:, :, 0], 0.01)   # no test rides on a near-zero uniform
    tau = {"greedy": 0.0, "mss": 0.8, "exec": 0.6}[rule]
    return logits, qd, parent, tok, unif, tau, spine


@pytest.mark.parametrize("V,ldt", [(20000, "bf16"), (65536, "bf16"), (20000, "f32")])
@pytest.mark.parametrize("rule", ["mss", "greedy", "exec"])
def test_chain_walks(V, ldt, rule):
    _say("accept chains V=%d %s %s" % (V, ldt, rule))
    logits, qd, parent, tok, unif, tau, spine = _spine(V, ldt, rule, seed=V + len(rule))
    ref = oracle.accept(logits, ldt, qd, parent, tok, unif, tau, trace=True)
    rp, rl, rb = ref[:3]
    # the case reaches what it is for: every walk goes down the whole spine
    assert np.all(rl == D + 1)
    for b in range(len(SWITCH)):
        assert np.array_equal(rp[b, :D + 1], spine[b])
    d = [dev_tensor(a) for a in (logits, parent, tok, unif)]
    dq = dev_tensor(qd) if qd is not None else None
    p, l, bo = tva.accept(d[0], dq, d[1], d[2], d[3], tau)
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    compare_accept((p.cpu().numpy(), l.cpu().numpy(), bo.cpu().numpy()), (rp, rl, rb), ref[3])
