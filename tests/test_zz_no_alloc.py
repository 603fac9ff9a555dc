"""sd_accept_commit_noalloc (no workspace, the library's own exchange slots)
against sd_accept_commit on the same inputs: path, length, bonus, committed
K/V and context lengths bit for bit, on two calls in a row, the second with
a smaller input, then on calls of the other two rules."""
import sys

import numpy as np
import pytest
import torch

from synth import CONFIGS, make_inputs, small_variant
from tests.devutil import to_device

tva = pytest.importorskip("tree_verification_amd")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _tau(c):
    return 0.0 if c.mode == "greedy" else c.temperature


def _bits(t):
    return t.view(torch.uint8).cpu().numpy() if t.dtype != torch.int32 else t.cpu().numpy()


def _both(c, x):
    """The workspace call and the no-allocation call, each on its own fresh
    copy of the inputs; returns both results as host arrays."""
    tau = _tau(c)
    res = []
    for fused in ("ws", "noalloc"):
        d = to_device(x)
        draft = d["draft"] if c.mode == "mss" else None
        if fused == "ws":
            p, l, b = tva.accept_commit(d["logits"], draft, d["parent"], d["token"], d["unif"], tau,
                                        d["k"], d["v"], d["table"], d["ctx"])
            torch.cuda.synchronize()
            st = tva.device_status()
        else:
            status = torch.zeros(1, dtype=torch.int32, device="cuda")
            p, l, b = tva.accept_commit_noalloc(d["logits"], draft, d["parent"], d["token"],
                                                d["unif"], tau, d["k"], d["v"], d["table"],
                                                d["ctx"], status)
            torch.cuda.synchronize()
            st = tva.device_status(ws=status)
        res.append(dict(path=p.cpu().numpy(), plen=l.cpu().numpy(), bonus=b.cpu().numpy(),
                        k=_bits(d["k"]), v=_bits(d["v"]), ctx=d["ctx"].cpu().numpy(), status=st))
        del d
    return res


def _same(a, b, where):
    for key in ("path", "plen", "bonus", "k", "v", "ctx", "status"):
        assert np.array_equal(a[key], b[key]), "%s: %s differs" % (where, key)


def test_noalloc_matches_workspace_call_twice_smaller_second():
    # first call: the benchmarked shape (16 sequences x 16 workgroups, 128256 tokens)
    c1 = CONFIGS["llama3_8b_tree64"]
    _say("noalloc call 1: %s" % c1.name)
    ws1, na1 = _both(c1, make_inputs(c1))
    _same(ws1, na1, "call 1")
    assert ws1["status"] == 0 and (ws1["plen"] >= 1).all()
    # second call, smaller: 3 sequences x 3 workgroups over a 4099-token vocabulary;
    # the slots the first call used must not leak into it
    c2 = small_variant("llama3_8b_tree64")
    _say("noalloc call 2: %s" % c2.name)
    ws2, na2 = _both(c2, make_inputs(c2))
    _same(ws2, na2, "call 2")
    assert ws2["status"] == 0


@pytest.mark.parametrize("name", ["specexec_70b_tree2048", "longctx_paged_tree16", "tiny_chain"])
def test_noalloc_other_rules(name):
    """Target sampling, rejection sampling over a shuffled table, and greedy
    with float32 logits and one workgroup per sequence."""
    c = small_variant(name)
    _say("noalloc %s" % c.name)
    ws, na = _both(c, make_inputs(c))
    _same(ws, na, name)


def test_noalloc_sets_status_bits():
    """A bad parent: the tree's sequence gets path length 0 and the bit goes
    to the caller's status word."""
    c = small_variant("llama3_8b_tree64")
    x = make_inputs(c)
    x.tree_parent[1, 5] = 7                      # parent after its child
    d = to_device(x)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    p, l, b = tva.accept_commit_noalloc(d["logits"], d["draft"], d["parent"], d["token"], d["unif"],
                                        c.temperature, d["k"], d["v"], d["table"], d["ctx"], status)
    torch.cuda.synchronize()
    assert int(l[1]) == 0
    assert tva.device_status(ws=status) & 0x1
    assert tva.device_status(ws=status) == 0     # read and cleared


def test_noalloc_many_sequences():
    """129 sequences: one workgroup each (a sequence spans several only when
    B <= 128, which the library's slots always cover), still equal to the
    workspace call."""
    c = small_variant("llama3_8b_tree64", B=129, V=1000)
    _say("noalloc %s B=129" % c.name)
    ws, na = _both(c, make_inputs(c))
    _same(ws, na, "B=129")
