"""sd_tree_build on the GPU against the oracle's sequential best-first search
(and, for the 2048-node workload, against the input generator's tree): the
parent and token arrays bit for bit, the cumulative log-probabilities to
1e-9."""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_inputs
from synth.inputs import _normals, _rng, S_DRAFT, f32_to_bf16_bits
from tests.devutil import dev_tensor

tva = pytest.importorskip("tree_verification_amd")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _build(stored, dt, tau, root=0):
    p, t, c, rounds = tva.tree_build(dev_tensor(stored), tau, root)
    torch.cuda.synchronize()
    assert tva.device_status() == 0
    return p.cpu().numpy(), t.cpu().numpy(), c.cpu().numpy(), rounds


def _check(stored, dt, tau, root=0):
    T = stored.shape[0]
    gp, gt, gc, rounds = _build(stored, dt, tau, root)
    # the C ABI takes the temperature as float32: the oracle divides by the same value
    rp, rt, rc = oracle.build_tree(stored, dt, float(np.float32(tau)), T, root)
    assert np.array_equal(gp, rp), "parent differs at %s" % np.nonzero(gp != rp)[0][:5]
    assert np.array_equal(gt, rt), "token differs at %s" % np.nonzero(gt != rt)[0][:5]
    assert np.abs(gc - rc).max() <= 1e-9
    return gp, gt, rounds


def test_build_specexec_tree_equals_generator():
    """The 2048-node best-first tree of the SpecExec-scale workload, from the
    same seeded drafter table (32000 tokens, N(0, 3^2)): equal to the input
    generator's tree and to the oracle's."""
    c = CONFIGS["specexec_70b_tree2048"]
    _say("tree build %d x %d" % (c.T, c.V))
    d = _normals(_rng(c, S_DRAFT), (c.T, c.V), c.logit_sigma, "f32")
    x = make_inputs(c)
    gp, gt, rounds = _check(d, "f32", 1.0, root=int(x.tree_token[0, 0]))
    assert np.array_equal(gp, x.tree_parent[0]) and np.array_equal(gt, x.tree_token[0])
    _say("rounds %d" % rounds)
    assert rounds < c.T


@pytest.mark.parametrize("T,V,tau,dt,seed", [(1, 700, 1.0, "f32", 0), (2, 700, 1.0, "f32", 1),
                                             (160, 700, 1.0, "f32", 2), (160, 700, 0.6, "bf16", 3),
                                             (50, 3, 1.0, "f32", 4), (512, 4099, 1.0, "bf16", 5),
                                             (1000, 32000, 0.8, "f32", 6)])
def test_build_random_tables(T, V, tau, dt, seed):
    """Shapes from one node to the workload's scale; a 3-token vocabulary (a
    round then has fewer candidates than the budget asks for); bf16 tables
    and temperatures other than 1."""
    _say("tree build T=%d V=%d tau=%g %s" % (T, V, tau, dt))
    rng = np.random.default_rng(seed)
    d = (rng.standard_normal((T, V)) * 3).astype(np.float32)
    stored = f32_to_bf16_bits(d) if dt == "bf16" else d
    _check(stored, dt, tau, root=seed % V)


def test_build_peaked_rows_many_rounds():
    """A drafter whose rows each favour one token strongly: most rounds can
    take only a node or two (the best child of a new node beats the other
    candidates), so the round loop runs long."""
    T, V = 96, 64
    rng = np.random.default_rng(9)
    d = rng.standard_normal((T, V)).astype(np.float32)
    d[np.arange(T), rng.integers(0, V, size=T)] += 8.0
    _say("tree build peaked")
    gp, gt, rounds = _check(d, "f32", 1.0)
    assert rounds > 10


def test_build_two_token_closed_form():
    """p = (0.9, 0.1) at every node: the root, a chain of 21 zeros, then the
    root's child 1 (0.9^21 > 0.1 > 0.9^22)."""
    T = 23
    d = np.tile(np.log(np.array([0.9, 0.1])), (T, 1)).astype(np.float32)
    gp, gt, gc, _ = _build(d, "f32", 1.0)
    assert list(gp[:22]) == [-1] + list(range(21)) and list(gt[1:22]) == [0] * 21
    assert gp[22] == 0 and gt[22] == 1


def test_build_workspace_reuse_across_shapes():
    """One workspace for a large build, then a small one, then the large again."""
    rng = np.random.default_rng(11)
    big = (rng.standard_normal((600, 5000)) * 3).astype(np.float32)
    small = (rng.standard_normal((40, 300)) * 3).astype(np.float32)
    for d in (big, small, big):
        _check(d, "f32", 1.0)
