"""sd_tree_expand on the GPU against the oracle: exact where float32 cannot
decide (integer logits at temperature 1, rows far apart), and elsewhere the
same set up to candidates within float32 error of the k-th score, output in
the order of the GPU's own scores."""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth.inputs import f32_to_bf16_bits
from tests.devutil import dev_tensor

tva = pytest.importorskip("tree_verification_amd")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(logits, dtype, cum, tau, k):
    d = dev_tensor(logits)
    if dtype == "bf16":
        d = d.view(torch.bfloat16)
    r, t, s = tva.tree_expand(d, dev_tensor(cum.astype(np.float32)), tau, k)
    torch.cuda.synchronize()
    return r.cpu().numpy(), t.cpu().numpy(), s.cpu().numpy()


def _check(gpu, logits, dtype, cum, tau, k):
    """The GPU's k picks against the oracle's scores of every candidate."""
    E, V = logits.shape
    r, t, s = gpu
    rr, rt, rs = oracle.expand(logits, dtype, cum, tau, E * V)
    full = np.empty(E * V)
    full[rr.astype(np.int64) * V + rt] = rs
    s_k = rs[k - 1]
    delta = 2e-5 * (1.0 + abs(s_k))
    flat = r.astype(np.int64) * V + t
    assert len(set(flat.tolist())) == k
    assert (full[flat] >= s_k - delta).all()
    clear = rr.astype(np.int64)[:k] * V + rt[:k]
    clear = clear[rs[:k] > s_k + delta]
    assert set(clear.tolist()) <= set(flat.tolist())
    assert np.allclose(s, full[flat], rtol=0, atol=delta)
    # best first by the GPU's own float32 scores, ties to the smaller flat index
    for i in range(k - 1):
        assert s[i] > s[i + 1] or (s[i] == s[i + 1] and flat[i] < flat[i + 1])


def test_single_row_integer_logits_exact():
    rng = np.random.default_rng(0)
    l = rng.integers(-6, 7, size=(1, 3000)).astype(np.float32)       # many exact ties
    _say("expand single row")
    r, t, s = _run(l, "f32", np.zeros(1), 1.0, 700)
    want = sorted(range(3000), key=lambda x: (-l[0, x], x))[:700]
    assert t.tolist() == want and (r == 0).all()


def test_rows_far_apart_exact():
    """Identical rows with cumulative log-probabilities 50 apart: every pick of
    row 0 beats row 1's, and inside a row the order is by logit, then token."""
    rng = np.random.default_rng(1)
    row = rng.integers(-20, 21, size=500).astype(np.float32)     # exact ties, gaps >> float32 error
    l = np.tile(row, (3, 1))
    cum = np.array([0.0, -50.0, -100.0])
    _say("expand rows far apart")
    r, t, s = _run(l, "f32", cum, 0.9, 1200)
    by_logit = sorted(range(500), key=lambda x: (-row[x], x))
    assert r.tolist() == [0] * 500 + [1] * 500 + [2] * 200
    assert t.tolist() == by_logit + by_logit + by_logit[:200]


@pytest.mark.parametrize("E,V,k,tau,dtype", [
    (64, 32000, 2048, 0.6, "bf16"),     # a batch of the 2048-node search's shape
    (16, 128256, 512, 0.8, "bf16"),
    (5, 1001, 4096, 1.0, "f32"),        # ragged vocabulary, k at its maximum
    (7, 333, 1, 0.5, "f32"),
    (1, 4096, 4096, 1.3, "bf16"),       # every candidate
    (256, 32000, 2048, 0.6, "bf16"),    # large batches: four chunks per workgroup
    (700, 12345, 1000, 0.9, "f32"),     # the same, ragged vocabulary
])
def test_expand_matches_oracle(E, V, k, tau, dtype):
    rng = np.random.default_rng(E * 7919 + V)
    l = (rng.standard_normal((E, V)) * 3).astype(np.float32)
    cum = -rng.random(E) * 5
    if dtype == "bf16":
        l = f32_to_bf16_bits(l)
    _say("expand E=%d V=%d k=%d %s" % (E, V, k, dtype))
    gpu = _run(l, dtype, cum, tau, k)
    _check(gpu, l, dtype, cum.astype(np.float32), tau, k)


def test_expand_workspace_reuse():
    rng = np.random.default_rng(5)
    l = (rng.standard_normal((8, 2000)) * 3).astype(np.float32)
    cum = -rng.random(8)
    a = _run(l, "f32", cum, 0.7, 300)
    b = _run(l, "f32", cum, 0.7, 300)
    c = _run(l, "f32", cum, 0.7, 17)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert np.array_equal(c[0], a[0][:17]) and np.array_equal(c[1], a[1][:17])


def test_expand_workspace_across_shapes():
    """One workspace for calls of different batch sizes and k in a row: each
    result matches the oracle (the counter and histograms do not move with
    the shape)."""
    for E, V, k in ((300, 2000, 900), (8, 2000, 50), (1000, 1500, 4096), (3, 777, 5)):
        rng = np.random.default_rng(E + 17)
        l = (rng.standard_normal((E, V)) * 3).astype(np.float32)
        cum = -rng.random(E) * 4
        _say("expand across shapes E=%d" % E)
        gpu = _run(l, "f32", cum, 0.8, k)
        _check(gpu, l, "f32", cum.astype(np.float32), 0.8, k)
